// HARP-style butterfly: log2(n) stages of 2x2 orthogonal blocks on pairs at
// stride 2^s, then a gather permutation; optional fused int4 quantization.
//
// Source: HARP abstract (product of sparse butterfly-like block-orthogonal
// stages) and HARP technical summary (gist.science) sections 2.1, 2.2, 2.4
// (block kernel Q(theta) G_2; stride stages applied without materialising the
// permutations -- here the pairs are addressed in place).
#include <math.h>

#include "hr_internal.h"
#include "hr_device.h"
#include "quant_lds.h"

namespace hr {

// One thread per (stage, pair): coefficients evaluated in double precision.
__global__ void butterfly_coeffs_kernel(const float* __restrict__ angles, int half, int total,
                                        int precondition, float2* __restrict__ coeffs) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const double th = (double)angles[idx];
  const double c = cos(th), t = sin(th);
  float2 out;
  if (precondition) {
    const double r = 0.70710678118654752440;  // 1/sqrt(2)
    out.x = (float)((c - t) * r);
    out.y = (float)((c + t) * r);
  } else {
    out.x = (float)c;
    out.y = (float)t;
  }
  coeffs[idx] = out;
}

hipError_t launch_butterfly_coeffs(const float* angles, int n, int log2n, int precondition,
                                   float* coeffs, hipStream_t s) {
  const int total = log2n * (n >> 1);
  const int threads = 256;
  hipLaunchKernelGGL(butterfly_coeffs_kernel, dim3((total + threads - 1) / threads), dim3(threads),
                     0, s, angles, n >> 1, total, precondition, reinterpret_cast<float2*>(coeffs));
  return hipGetLastError();
}

constexpr int kBfThreads = 256;

// Apply the block of pair (i, j): rotation [[c,-t],[t,c]] (stored (c,t)) or
// reflection-form [[u,v],[v,-u]] (stored (u,v)); TRANSPOSE applies the
// transposed block (the reflection form is symmetric).
template <bool PRECOND, bool TRANSPOSE>
__device__ __forceinline__ void apply_block(float& a, float& b, float2 k) {
  const float u = a, v = b;
  if (PRECOND) {
    a = k.x * u + k.y * v;
    b = k.y * u - k.x * v;
  } else if (!TRANSPOSE) {
    a = k.x * u - k.y * v;
    b = k.y * u + k.x * v;
  } else {
    a = k.x * u + k.y * v;
    b = -k.y * u + k.x * v;
  }
}

template <bool PRECOND, bool INVERSE>
__global__ __launch_bounds__(kBfThreads) void butterfly_generic_kernel(ButterflyArgs a) {
  extern __shared__ float sm[];  // 2n floats: working row + permutation staging
  float* z = sm;
  float* t2 = sm + a.n;
  const int tid = threadIdx.x;
  const int n = a.n, L = a.log2n, half = n >> 1;
  const float2* co = reinterpret_cast<const float2*>(a.coeffs);
  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const float* xr = a.x + row * n;
    if (!INVERSE) {
      for (int i = tid; i < n; i += kBfThreads) z[i] = xr[i];
    } else {
      for (int i = tid; i < n; i += kBfThreads) z[a.perm ? a.perm[i] : i] = xr[i];
    }
    __syncthreads();
    for (int k = 0; k < L; ++k) {
      const int st = INVERSE ? (L - 1 - k) : k;
      const int h = 1 << st;
      for (int t = tid; t < half; t += kBfThreads) {
        const int i = ((t >> st) << (st + 1)) | (t & (h - 1));
        float u = z[i], v = z[i + h];
        apply_block<PRECOND, INVERSE>(u, v, co[st * half + t]);
        z[i] = u;
        z[i + h] = v;
      }
      __syncthreads();
    }
    const float* out = z;
    if (!INVERSE && a.perm) {
      for (int i = tid; i < n; i += kBfThreads) t2[i] = z[a.perm[i]];
      __syncthreads();
      out = t2;
    }
    if (a.y) {
      float* yr = a.y + row * n;
      for (int i = tid; i < n; i += kBfThreads) yr[i] = out[i];
    }
    if (a.codes) {
      quant_row_from_lds(out, 1.0f, n, a.group, a.codes + row * (n >> 1), a.scales,
                         row * (n / a.group), a.scale_f16);
    }
    __syncthreads();
  }
}

hipError_t launch_butterfly(const ButterflyArgs& a, hipStream_t s) {
  if (launch_butterfly4096(a, s)) return hipGetLastError();
  const int64_t grid64 = a.rows < 4096 ? a.rows : 4096;
  const dim3 grid((unsigned)grid64), block(kBfThreads);
  const size_t lds = 2 * sizeof(float) * (size_t)a.n;
  if (a.precondition) {
    if (a.inverse) hipLaunchKernelGGL((butterfly_generic_kernel<true, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((butterfly_generic_kernel<true, false>), grid, block, lds, s, a);
  } else {
    if (a.inverse) hipLaunchKernelGGL((butterfly_generic_kernel<false, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((butterfly_generic_kernel<false, false>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace hr
