// Rotation setup: quaternion pairs -> SO(4) block matrices.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract (block-diagonal SO(4) rotations, 256
// stored parameters per head) and FreeToken issue #141, Proposed Solution
// (quaternion rotations).  Block b maps v = v0 + v1 i + v2 j + v3 k to
// a * v * conj(p), a and p the normalised quaternions.  As a matrix that is
// L(a) R(conj(p)), L and R the left- and right-multiplication matrices.
#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

__global__ void rotation_init_kernel(const float* __restrict__ quats, int n, float* __restrict__ rot) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // (head, block)
  if (i >= n) return;
  double a[4], p[4];
  double na = 0, np = 0;
  for (int k = 0; k < 4; ++k) {
    a[k] = quats[i * 8 + k];
    p[k] = quats[i * 8 + 4 + k];
    na += a[k] * a[k];
    np += p[k] * p[k];
  }
  na = 1.0 / sqrt(na);
  np = 1.0 / sqrt(np);
  for (int k = 0; k < 4; ++k) { a[k] *= na; p[k] *= np; }
  // r = conj(p)
  const double r0 = p[0], r1 = -p[1], r2 = -p[2], r3 = -p[3];
  const double L[4][4] = {{a[0], -a[1], -a[2], -a[3]},
                          {a[1], a[0], -a[3], a[2]},
                          {a[2], a[3], a[0], -a[1]},
                          {a[3], -a[2], a[1], a[0]}};
  const double R[4][4] = {{r0, -r1, -r2, -r3},
                          {r1, r0, r3, -r2},
                          {r2, -r3, r0, r1},
                          {r3, r2, -r1, r0}};
  for (int row = 0; row < 4; ++row)
    for (int col = 0; col < 4; ++col) {
      double s = 0;
      for (int k = 0; k < 4; ++k) s += L[row][k] * R[k][col];
      rot[i * 16 + row * 4 + col] = (float)s;
    }
}

hipError_t launch_rotation_init(const float* quats_dev, int hkv, float* rot_dev, hipStream_t stream) {
  const int n = hkv * kBlocks;
  hipLaunchKernelGGL(rotation_init_kernel, dim3((n + 127) / 128), dim3(128), 0, stream, quats_dev,
                     n, rot_dev);
  return hipGetLastError();
}

}  // namespace iq
