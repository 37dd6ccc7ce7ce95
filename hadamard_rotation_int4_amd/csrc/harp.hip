// HARP's general processor: mixed-radix stages of dense b x b orthogonal
// blocks B_{t,c} = Q_{t,c}(theta) G_{b_t} (HARP technical summary, sections
// 2.1 and 2.2: a schedule b = (b_0 .. b_{m-1}) with prod b_t = d, stages of
// block-diagonal orthogonal matrices separated by stride permutations; Q a
// Givens rotation for b = 2 and the Cayley map for b > 2; G the normalised
// Sylvester-Hadamard matrix for powers of two, a fixed QR fallback otherwise).
//
// Indexing: coordinate i = sum_t i_t S_t with S_t = b_0 ... b_{t-1}.  Stage t
// acts along digit t; block c = lo + S_t hi holds coordinates
// lo + S_t (r + b_t hi), r < b_t, and maps them by y_r = sum_q B[c][r][q] x_q.
// The stride permutations are folded into this addressing.
//
// harp_blocks_kernel: one thread per block, in double precision: Q (Givens,
// or Gauss-Jordan solve of (I - A) Q = I + A), times G, stored as fp32.  The
// table is coefficient-major per stage, [b][b][d/b]: coefficient (r, q) of
// block c at (r b + q) d/b + c, so the lanes of a wave, which own consecutive
// blocks, read each coefficient as one contiguous 256-byte run.
// harp_apply_kernel: a persistent workgroup keeps R rows in LDS and runs
// every stage over them; each thread takes blocks c = tid, tid + 1024, ...,
// holds the block's b^2 coefficients in registers while it maps that block of
// all R rows, so the coefficient table (d * sum b_t floats, read from L2) is
// fetched once per R rows.  Quantization (int4, per group) is fused at the end.
#include "hr_internal.h"
#include "hr_device.h"
#include "quant_lds.h"

namespace hr {

// 1024 threads: the radix-8 stages of d = 5120 (640 blocks) and its radix-5
// stage (1024 blocks) each take one round (with 512 threads the radix-8 stages took two rounds: 96 us against 89 us)
constexpr int kHarpThreads = 1024;

// LDS position of in-row element i when 64 divides d: bits 2-5 XORed with
// bits 6-9 of i, a permutation inside every aligned block of 64 elements.
// The stride-S gathers of the 5120 schedule then put at most 4, 2, 1, 1, 1
// lanes on a bank (stages 0 .. 4), against 8, 8, 1, 1, 1 unswizzled; groups
// of 4 stay contiguous, so rows still move as float4.
__device__ __forceinline__ int hswz(int i, bool on) { return on ? i ^ (((i >> 6) & 15) << 2) : i; }
struct HarpPos {
  bool on;
  __device__ int operator()(int i) const { return hswz(i, on); }
};

__device__ __forceinline__ bool hp_pow2(int b) { return (b & (b - 1)) == 0; }

// one thread per block of every stage
__global__ __launch_bounds__(256) void harp_blocks_kernel(HarpSchedule sc, const float* __restrict__ theta,
                                                          const float* __restrict__ fallbacks,
                                                          float* __restrict__ blocks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int t = 0;
  while (t < sc.nstages && gid >= sc.block_begin[t + 1]) ++t;
  if (t >= sc.nstages) return;
  const int b = sc.radix[t];
  const int64_t c = gid - sc.block_begin[t];
  const int P = b == 2 ? 1 : b * (b - 1) / 2;
  const float* th = theta + sc.theta_off[t] + c * P;
  double q[kHarpMaxRadix][kHarpMaxRadix];
  if (b == 2) {
    const double a = (double)th[0];
    const double cs = cos(a), sn = sin(a);
    q[0][0] = cs; q[0][1] = -sn;
    q[1][0] = sn; q[1][1] = cs;
  } else {
    // (I - A) Q = (I + A), A skew-symmetric from the upper-triangle parameters;
    // Gauss-Jordan with partial pivoting on [I - A | I + A]
    double m[kHarpMaxRadix][kHarpMaxRadix], r[kHarpMaxRadix][kHarpMaxRadix];
    for (int i = 0; i < b; ++i)
      for (int j = 0; j < b; ++j) { m[i][j] = i == j ? 1.0 : 0.0; r[i][j] = m[i][j]; }
    int k = 0;
    for (int i = 0; i < b; ++i)
      for (int j = i + 1; j < b; ++j, ++k) {
        const double a = (double)th[k];
        m[i][j] -= a; m[j][i] += a;      // I - A
        r[i][j] += a; r[j][i] -= a;      // I + A
      }
    for (int col = 0; col < b; ++col) {
      int piv = col;
      for (int i = col + 1; i < b; ++i)
        if (fabs(m[i][col]) > fabs(m[piv][col])) piv = i;
      if (piv != col)
        for (int j = 0; j < b; ++j) {
          double u = m[col][j]; m[col][j] = m[piv][j]; m[piv][j] = u;
          u = r[col][j]; r[col][j] = r[piv][j]; r[piv][j] = u;
        }
      const double inv = 1.0 / m[col][col];
      for (int j = 0; j < b; ++j) { m[col][j] *= inv; r[col][j] *= inv; }
      for (int i = 0; i < b; ++i) {
        if (i == col) continue;
        const double f = m[i][col];
        if (f == 0.0) continue;
        for (int j = 0; j < b; ++j) { m[i][j] -= f * m[col][j]; r[i][j] -= f * r[col][j]; }
      }
    }
    for (int i = 0; i < b; ++i)
      for (int j = 0; j < b; ++j) q[i][j] = r[i][j];
  }
  // B = Q G
  const float* fb = fallbacks + sc.fallback_off[t];
  const double nrm = 1.0 / sqrt((double)b);
  const int64_t nb = sc.block_begin[t + 1] - sc.block_begin[t];
  float* out = blocks + sc.blocks_off[t] + c;
  for (int i = 0; i < b; ++i)
    for (int j = 0; j < b; ++j) {
      double s = 0.0;
      for (int l = 0; l < b; ++l) {
        const double g = hp_pow2(b) ? ((__builtin_popcount(l & j) & 1) ? -nrm : nrm)
                                    : (double)fb[l * b + j];
        s += q[i][l] * g;
      }
      out[(int64_t)(i * b + j) * nb] = (float)s;
    }
}

// Map every block c of one stage (radix B) over the R rows in LDS.
template <int B>
__device__ __forceinline__ void harp_stage(float* lds, int d, int R, int S, int nb,
                                           const float* __restrict__ blk, bool inverse, bool swz) {
  for (int c = threadIdx.x; c < nb; c += kHarpThreads) {
    float m[B][B];
    const float* src = blk + c;
    if (inverse) {
#pragma unroll
      for (int i = 0; i < B; ++i)
#pragma unroll
        for (int j = 0; j < B; ++j) m[i][j] = src[(int64_t)(j * B + i) * nb];
    } else {
#pragma unroll
      for (int i = 0; i < B; ++i)
#pragma unroll
        for (int j = 0; j < B; ++j) m[i][j] = src[(int64_t)(i * B + j) * nb];
    }
    const int lo = c % S, hi = c / S;
    const int base = lo + S * B * hi;
    int pos[B];
#pragma unroll
    for (int q = 0; q < B; ++q) pos[q] = hswz(base + q * S, swz);
    for (int r = 0; r < R; ++r) {
      float* row = lds + r * d;
      float v[B];
#pragma unroll
      for (int q = 0; q < B; ++q) v[q] = row[pos[q]];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int q = 0; q < B; ++q) acc = fmaf(m[i][q], v[q], acc);
        row[pos[i]] = acc;
      }
    }
  }
}

__global__ __launch_bounds__(kHarpThreads) void harp_apply_kernel(HarpArgs a) {
  extern __shared__ float lds[];
  const int d = a.d, R = a.rows_per_group;
  const int tid = threadIdx.x;
  const bool swz = (d & 63) == 0;
  const int64_t ngroups = (a.rows + R - 1) / R;
  for (int64_t rg = blockIdx.x; rg < ngroups; rg += gridDim.x) {
    const int64_t r0 = rg * R;
    const int nr = (int)(a.rows - r0 < R ? a.rows - r0 : R);
    // load nr rows (float4; d is a multiple of 4)
    const int q4 = d / 4;
    for (int i = tid; i < nr * q4; i += kHarpThreads) {
      const int r = i / q4, k = i - r * q4;
      *reinterpret_cast<float4*>(lds + r * d + hswz(4 * k, swz)) =
          reinterpret_cast<const float4*>(a.x + (r0 + r) * d)[k];
    }
    __syncthreads();
    for (int s = 0; s < a.sc.nstages; ++s) {
      const int t = a.inverse ? a.sc.nstages - 1 - s : s;
      const int b = a.sc.radix[t], S = a.sc.stride[t], nb = d / b;
      const float* blk = a.blocks + a.sc.blocks_off[t];
      switch (b) {
        case 2: harp_stage<2>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        case 3: harp_stage<3>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        case 4: harp_stage<4>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        case 5: harp_stage<5>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        case 6: harp_stage<6>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        case 7: harp_stage<7>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
        default: harp_stage<8>(lds, d, nr, S, nb, blk, a.inverse, swz); break;
      }
      __syncthreads();
    }
    if (a.y) {
      for (int i = tid; i < nr * q4; i += kHarpThreads) {
        const int r = i / q4, k = i - r * q4;
        reinterpret_cast<float4*>(a.y + (r0 + r) * d)[k] =
            *reinterpret_cast<const float4*>(lds + r * d + hswz(4 * k, swz));
      }
    }
    if (a.codes) quant_rows_from_lds(lds, d, nr, d, a.group, a.codes, r0, a.scales, a.scale_f16, HarpPos{swz});
    __syncthreads();
  }
}

hipError_t launch_harp_blocks(const HarpSchedule& sc, const float* theta, const float* fallbacks,
                              float* blocks, hipStream_t s) {
  const int64_t total = sc.block_begin[sc.nstages];
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(harp_blocks_kernel, dim3((unsigned)grid), dim3(256), 0, s, sc, theta, fallbacks,
                     blocks);
  return hipGetLastError();
}

hipError_t launch_harp_apply(HarpArgs a, hipStream_t s) {
  // as many rows per group as fit in 160 KB of LDS (at most 8), one
  // workgroup per CU: every group re-reads the whole coefficient table from
  // L2, which outweighs overlapping two workgroups' loads with each other's
  // stages (d = 5120: 8 rows per group, 96 us, against 3 rows and two
  // workgroups, 120 us)
  int R = (int)(40960 / a.d);
  if (R > 8) R = 8;
  if (R < 1) R = 1;
  a.rows_per_group = R;
  const int64_t ngroups = (a.rows + R - 1) / R;
  const int64_t grid = ngroups < 512 ? ngroups : 512;
  const size_t lds = sizeof(float) * (size_t)R * a.d;
  // more than 64 KB of dynamic LDS must be allowed explicitly (160 KB per
  // workgroup on gfx950)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(harp_apply_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(harp_apply_kernel, dim3((unsigned)grid), dim3(kHarpThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace hr
