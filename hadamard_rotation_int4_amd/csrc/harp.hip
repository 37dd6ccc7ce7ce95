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
// table is quad-major per stage, [ceil(b^2 / 4)][d/b][4]: coefficient k =
// r b + q of block c at ((k / 4) d/b + c) 4 + k % 4 (the last quad padded with
// zeros), so a thread loads its block's coefficients four at a time and the
// lanes of a wave, which own consecutive blocks, read each quad as one
// contiguous 1 KB run (four times fewer load instructions than one
// coefficient per load: fp32 4096 x 5120, same box, 70.6 against 55.2 us
// with no coefficient loads at all).
// harp_apply_kernel: a persistent workgroup keeps R rows in LDS (loaded by
// LDS-DMA, every load in flight at once) and runs every stage over them; each
// thread takes blocks c = tid, tid + 1024, ..., holds the block's b^2
// coefficients in registers while it maps that block of all R rows, so the
// coefficient table (d * sum b_t floats, read from L2) is fetched once per R
// rows, and requests its first block's coefficients before the barrier that
// opens the stage.  Quantization (int4, per group) is fused at the end.
#include "hr_internal.h"
#include "hr_device.h"
#include "quant_lds.h"

namespace hr {

// 1024 threads: the radix-8 stages of d = 5120 (640 blocks) and its radix-5
// stage (1024 blocks) each take one round (with 512 threads the radix-8 stages took two rounds: 96 us against 89 us)
constexpr int kHarpThreads = 1024;

// 16-byte global -> LDS copy (LDS-DMA: lane i's 16 bytes land at lp + 16 i)
// nt: with the nontemporal hint.  Measured on fp32 4096 x 5120, two buffer
// sets in turn, same box: with fp32 output 82.0 -> 75.5 us, with int4 codes
// 85.9 -> 87.5 us, so only the fp32 output of a streamed input takes it.
__device__ __forceinline__ void harp_lds_load16(const void* gp, void* lp, bool nt) {
  if (nt) __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 2);
  else __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}

// LDS position of in-row element i when 64 divides d: with x = bits 6-9 of
// i, bits 2-5 XORed with t(x) = (x & 1) | ((x & 7) << 1), then bit 5 of the
// result XORed into bit 2.  Both steps permute each aligned block of 64
// elements, keep groups of 4 whole (rows move as float4) and are their own
// inverses, so the inverse applies them in reverse order.  A 4-byte access is
// served 32 lanes at a time over 32 banks, a 16-byte one 8 lanes at a time
// over 8 16-byte bank groups.  For the schedules of radix-8 stages (5120 =
// (8, 8, 8, 5, 2), 4096, 16384, ...) every stage's stride-S element accesses
// then reach 32 different banks per half-wave and 64 per wave, and every
// 16-byte access (the contiguous blocks of a stride-1 stage, the output copy,
// the quantizer's reads) 8 different groups per 8 lanes and 16 per 16.  (The
// first swizzle, bits 2-5 XORed with x ^ ((x & 1) << 3) alone, left 2 lanes
// to a bank in every half-wave of the stride-8 stage and 2 lanes to a group
// in the 16-byte reads of pieces 2i.)
__device__ __forceinline__ int hswz(int i, bool on) {
  const int x = (i >> 6) & 15;
  const int j = i ^ (((x & 1) | ((x & 7) << 1)) << 2);
  return on ? j ^ ((j >> 3) & 4) : i;
}
__device__ __forceinline__ int hswz_inv(int k, bool on) {
  const int j = k ^ ((k >> 3) & 4);
  const int x = (j >> 6) & 15;
  return on ? j ^ (((x & 1) | ((x & 7) << 1)) << 2) : k;
}
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
  float* out = blocks + sc.blocks_off[t] + 4 * c;
  for (int i = 0; i < b; ++i)
    for (int j = 0; j < b; ++j) {
      double s = 0.0;
      for (int l = 0; l < b; ++l) {
        const double g = hp_pow2(b) ? ((__builtin_popcount(l & j) & 1) ? -nrm : nrm)
                                    : (double)fb[l * b + j];
        s += q[i][l] * g;
      }
      const int k = i * b + j;
      out[(int64_t)(k >> 2) * nb * 4 + (k & 3)] = (float)s;
    }
  for (int k = b * b; k < 4 * ((b * b + 3) / 4); ++k) out[(int64_t)(k >> 2) * nb * 4 + (k & 3)] = 0.0f;
}

// The b^2 coefficients of block c (transposed for the inverse), loaded four
// at a time from the quad-major table.
template <int B>
__device__ __forceinline__ void harp_coeffs(float (&m)[B][B], const float* __restrict__ blk, int c, int nb,
                                            bool inverse) {
  constexpr int K4 = (B * B + 3) / 4;
  const float4* src = reinterpret_cast<const float4*>(blk) + c;
  float v[4 * K4];
#pragma unroll
  for (int k = 0; k < K4; ++k) {
    const float4 f = src[(int64_t)k * nb];
    v[4 * k] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
#pragma unroll
  for (int i = 0; i < B; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j) m[i][j] = inverse ? v[j * B + i] : v[i * B + j];
}

// Map block c of one stage over the R rows in LDS.
template <int B>
__device__ __forceinline__ void harp_block(const float (&m)[B][B], float* lds, int d, int R, int S, int c,
                                           bool swz) {
  const int lo = c % S, hi = c / S;
  const int base = lo + S * B * hi;
  if constexpr (B % 4 == 0) {
    if (S == 1 && (d & 3) == 0) {
      // contiguous block: B / 4 float4 pieces (whole under the swizzle)
      int p4[B / 4];
#pragma unroll
      for (int j = 0; j < B / 4; ++j) p4[j] = hswz(base + 4 * j, swz);
      for (int r = 0; r < R; ++r) {
        float* row = lds + r * d;
        float v[B];
#pragma unroll
        for (int j = 0; j < B / 4; ++j) {
          const float4 x = *reinterpret_cast<const float4*>(row + p4[j]);
          v[4 * j] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
        }
        float o[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
          float acc = 0.0f;
#pragma unroll
          for (int q = 0; q < B; ++q) acc = fmaf(m[i][q], v[q], acc);
          o[i] = acc;
        }
#pragma unroll
        for (int j = 0; j < B / 4; ++j)
          *reinterpret_cast<float4*>(row + p4[j]) = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
      }
      return;
    }
  }
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

// One stage (radix B) over the R rows in LDS.  A thread's first block's
// coefficients are requested before the barrier that ends the previous stage
// (or the row loads), so their L2 latency overlaps the other waves' work
// (prefetching the further blocks of b = 2 as well measured no faster).
template <int B>
__device__ __forceinline__ void harp_stage(float* lds, int d, int R, int S, int nb,
                                           const float* __restrict__ blk, bool inverse, bool swz) {
  const int c0 = threadIdx.x;
  float m[B][B];
  if (c0 < nb) harp_coeffs<B>(m, blk, c0, nb, inverse);
  __syncthreads();
  if (c0 < nb) harp_block<B>(m, lds, d, R, S, c0, swz);
  for (int c = c0 + kHarpThreads; c < nb; c += kHarpThreads) {
    harp_coeffs<B>(m, blk, c, nb, inverse);
    harp_block<B>(m, lds, d, R, S, c, swz);
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
    // load nr rows (float4; d is a multiple of 4) by LDS-DMA, 1 KB of LDS
    // per instruction and no registers held: LDS float4 p (row r, in-row k)
    // takes the row's float4 whose swizzled place is k; every load is in
    // flight before the barrier's wait
    const int q4 = d / 4, npc = nr * q4;
    const int wv = tid >> 6, ln = tid & 63;
    const float4* src = reinterpret_cast<const float4*>(a.x + r0 * d);
    for (int u = wv; u * 64 < npc; u += kHarpThreads / 64) {
      const int p = 64 * u + ln;
      if (p < npc) {
        const int r = p / q4, k = p - r * q4;
        harp_lds_load16(src + r * q4 + (hswz_inv(4 * k, swz) >> 2), lds + 256 * u, a.stream != 0);
      }
    }
    // (each stage starts with the barrier that waits for these loads or the
    // previous stage's writes)
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
    }
    __syncthreads();
    if (a.y) {
      for (int i = tid; i < npc; i += kHarpThreads) {
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
  // the row loads fill LDS in whole 1 KB runs: keep the rounded-up group
  // inside the 160 KB
  while (R > 1 && ((int64_t)R * a.d + 255) / 256 * 256 > 40960) --R;
  if (R < 1) R = 1;
  a.rows_per_group = R;
  a.stream = a.codes == nullptr && a.rows * a.d * 4 >= kStreamBytes;
  const int64_t ngroups = (a.rows + R - 1) / R;
  const int64_t grid = ngroups < 512 ? ngroups : 512;
  const size_t lds = sizeof(float) * (((size_t)R * a.d + 255) / 256 * 256);
  // more than 64 KB of dynamic LDS must be allowed explicitly (160 KB per
  // workgroup on gfx950)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(harp_apply_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(harp_apply_kernel, dim3((unsigned)grid), dim3(kHarpThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace hr
