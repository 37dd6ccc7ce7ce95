// Online rotation in the decode GEMM: y = H_K (d * x) / sqrt(K) of every
// activation row, int4 group quantization of y, and C = A W^T on the codes,
// in one kernel.
//
// What is computed: the randomized Hadamard transform and per-group int4
// quantization of hr_rotate_quant_int4 ("Experiment -- Hadamard rotation for
// int4 (W4A4) accuracy", Hypothesis and Method) followed by the W4A4 GEMM of
// hr_w4a4_gemm (same page, Hypothesis and Verdict: the per-group work stays
// inside one kernel).  The HARP technical summary (gist.science), section 4,
// puts the decode cost of an online processor at 0.0078 s against 0.0070 s
// per token; section 2.4 describes fused GPU kernels for its stages.  Here the
// rotated codes never go to memory between the two steps.
//
// Decode shape: M <= 16 rows of bf16 activations, K = 2048 or 4096.  Every
// workgroup (16 waves, 16 output columns) first rotates and quantizes all M
// rows into LDS -- wave w takes row w with the matrix-core transform of
// mfma2048.h (K = 4096 as two chunks and a lane-local H_2) and the same group
// quantizer as the rotation kernel -- then runs the decode GEMM loop of
// gemm_mfma.hip with A read from that resident buffer.  The first W loads are
// issued before the rotation, so they stream in while it runs.
//
// LDS layout of the codes: a run is 128 codes (64 bytes) of a row; run R's 16
// rows take 1 KB.  Row r, 16-byte piece p of run R sits at
//   R * 1024 + 64 * (r ^ (R & 3)) + 16 * (p ^ ((r >> 2) & 3) ^ ((R >> 2) & 3)).
// A rotating wave writes one dword per (run, piece): its 64 lanes cover 16
// runs (R & 15 distinct) x 4 dwords, and the two XORs put them on 64 distinct
// banks.  The GEMM lanes read 16 rows x 4 positions of one piece pair, which
// the XORs only permute within the run.
#include <type_traits>

#include "mfma2048.h"

namespace hr {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kFdWaves = 16;
constexpr int kFdRuns = 2;   // W runs per wave and chunk

__device__ __forceinline__ void fd_lds_load16(const void* gp, void* lp) {
  __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}

__device__ __forceinline__ uint32_t fd_a_off(int run, int row, int piece) {
  return (uint32_t)run * 1024u + 64u * (uint32_t)(row ^ (run & 3)) +
         16u * (uint32_t)(piece ^ ((row >> 2) & 3) ^ ((run >> 2) & 3));
}

template <int G, bool F16, int CH>
__global__ __launch_bounds__(kFdWaves * 64) void rotate_quant_gemm_decode_kernel(FusedDecodeArgs g) {
  constexpr int P = 2048;
  constexpr int K = CH * P;
  constexpr int RUNS = K / 128;
  constexpr int NG = K / G;
  constexpr int CR = kFdRuns;
  constexpr int MPG = G >= 64 ? G / 64 : 1;      // MFMAs per group (G = 32: one 16x16x32)
  constexpr int RPU = G >= 128 ? G / 128 : 1;    // runs per unit of work
  constexpr int GPC = G >= 64 ? 2 * CR / MPG : 4 * CR;   // groups per chunk
  typedef typename std::conditional<F16, _Float16, float>::type scale_t;
  __shared__ __attribute__((aligned(16))) char a_lds[RUNS * 1024];
  __shared__ __attribute__((aligned(16))) float sa_lds[NG][16];          // [group][row]
  __shared__ __attribute__((aligned(16))) uint4 stage_w[kFdWaves][CR][64];
  __shared__ float part[kFdWaves][16 * 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t rowb = K / 2;
  const int units = RUNS / RPU;
  const int rbeg = RPU * (wave * units / kFdWaves), rend = RPU * ((wave + 1) * units / kFdWaves);
  const bool arow = r < g.M;
  const int lrow = lane >> 2, lpiece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint8_t* lw = g.w + (n0 + lrow) * rowb + 16 * lpiece;
  auto issue_w = [&](int r0, int nr) {
#pragma unroll
    for (int t = 0; t < CR; ++t) {
      const int64_t run = r0 + (t < nr ? t : nr - 1);
      fd_lds_load16(lw + run * 64, &stage_w[wave][t][0]);
    }
  };
  // the first chunk of W is in flight during the rotation
  if (rbeg < rend) issue_w(rbeg, rend - rbeg < CR ? rend - rbeg : CR);

  // ---- rotation and quantization of row `wave` into LDS
  if (wave < g.M) {
    Mfma2048 Mt[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) mfma2048_init(Mt[c], lane, g.signs ? g.signs + c * P : nullptr);
    const int gq = Mt[0].g, a4 = Mt[0].a4;
    const float tau = Mt[0].tau;
    // lane (q, gq) holds, for K-step s, the 8 elements 128 A(q) + 8 gq + 32 s
    const uint16_t* xr = g.x + (int64_t)wave * K + 128 * a4 + 8 * gq;
    u32x4 b[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int s = 0; s < 4; ++s) b[c][s] = *reinterpret_cast<const u32x4*>(xr + c * P + 32 * s);
    f32x4 acc[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) mfma2048_transform(Mt[c], b[c], acc[c]);
    if (CH == 2) {
      // H_2 across the two chunks: same lane, same position, same sign tau
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f32x4 u0 = acc[0][t], u1 = acc[CH - 1][t];
        acc[0][t] = u0 + u1;
        acc[CH - 1][t] = u0 - u1;
      }
    }
    const float norm = g.norm;   // 1/sqrt(K)
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      // acc[ch][T][v] = tau * Y[a4][c], c = v + 4 T0 + 8 gq + 32 T1 + 64 T2: run m
      // (outputs 32 m + 8 gq + 0..7 of block a4) is tiles 2 m, 2 m + 1
      float mr[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 lo = acc[ch][2 * m], hi = acc[ch][2 * m + 1];
        const float m1 = fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])), fabsf(lo[2]));
        const float m2 = fmaxf(fmaxf(fabsf(lo[3]), fabsf(hi[0])), fabsf(hi[1]));
        const float m3 = fmaxf(fmaxf(m1, fabsf(hi[2])), fabsf(hi[3]));
        mr[m] = fmaxf(m2, m3);
      }
      constexpr int NL = G == 32 ? 4 : G == 64 ? 2 : 1;   // groups per lane
      float mg[NL];
      if (G == 32) {
#pragma unroll
        for (int m = 0; m < 4; ++m) mg[m] = mr[m];
      } else if (G == 64) {
        mg[0] = fmaxf(mr[0], mr[1]);
        mg[NL - 1] = fmaxf(mr[2], mr[3]);
      } else {
        mg[0] = fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3]));
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) mg[i] = max_over_rows(mg[i]);
      if (G == 256) mg[0] = __uint_as_float(umax_dpp<kQuadXor1>(__float_as_uint(mg[0])));
      float kk[NL], upv[NL];
      float s_own = 0.0f, s_own32 = 0.0f;
      bool need_clamp = false, need_up = false;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float s32 = div_const<7>(mg[i] * norm);
        const float s = F16 ? (float)(_Float16)s32 : s32;
        // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
        // values and scale are then both taken x 2^64 (exact; same quotients)
        upv[i] = (!F16 && s < 0x1p-100f) ? 0x1p64f : 1.0f;
        need_up |= !F16 && s > 0.0f && s < 0x1p-100f;
        kk[i] = s > 0.0f ? norm * __builtin_amdgcn_rcpf(s * upv[i]) * tau : 0.0f;
        need_clamp |= s > 0.0f && s < (F16 ? 6.103515625e-05f : 1.17549435e-38f);
        if (NL == 1 || i == (gq & (NL - 1))) {
          s_own = s;
          s_own32 = s32;
        }
      }
      // this lane's group (the same choice as the rotation kernel's scale store)
      int gi = -1;
      if (G == 32) gi = 4 * a4 + gq;
      else if (G == 64) gi = gq < 2 ? 2 * a4 + gq : -1;
      else if (G == 128) gi = gq == 0 ? a4 : -1;
      else gi = (gq == 0 && (a4 & 1) == 0) ? (a4 >> 1) : -1;
      if (gi >= 0) {
        gi += ch * (P / G);
        sa_lds[gi][wave] = s_own;
        if (g.a_scales && blockIdx.x == 0) {
          if (F16) reinterpret_cast<_Float16*>(g.a_scales)[(int64_t)wave * NG + gi] = (_Float16)s_own32;
          else reinterpret_cast<float*>(g.a_scales)[(int64_t)wave * NG + gi] = s_own32;
        }
      }
      const bool clamp = __builtin_amdgcn_ballot_w64(need_clamp) != 0;
      const bool tiny = !F16 && __builtin_amdgcn_ballot_w64(need_up) != 0;
      const float Mq = 12582920.0f;   // 1.5 * 2^23 + 8: the code, biased by 8, in the low bits
      const int run = ch * 16 + a4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int gl = G == 32 ? m : G == 64 ? (m >> 1) : 0;
        const float kx = kk[gl];
        f32x4 lo = acc[ch][2 * m], hi = acc[ch][2 * m + 1];
        if (tiny) {
          lo *= upv[gl];
          hi *= upv[gl];
        }
        float rr[8] = {fmaf(lo[0], kx, Mq), fmaf(lo[1], kx, Mq), fmaf(lo[2], kx, Mq), fmaf(lo[3], kx, Mq),
                       fmaf(hi[0], kx, Mq), fmaf(hi[1], kx, Mq), fmaf(hi[2], kx, Mq), fmaf(hi[3], kx, Mq)};
        if (clamp) {
#pragma unroll
          for (int e = 0; e < 8; ++e) rr[e] = __builtin_amdgcn_fmed3f(rr[e], Mq - 7.0f, Mq + 7.0f);
        }
        const uint32_t cw = pack8(rr);
        *reinterpret_cast<uint32_t*>(a_lds + fd_a_off(run, wave, m) + 4 * gq) = cw;
        if (g.a_codes && blockIdx.x == 0)
          reinterpret_cast<uint32_t*>(g.a_codes + (int64_t)wave * rowb)[(ch * P + 128 * a4 + 32 * m + 8 * gq) / 8] = cw;
      }
    }
  } else {
    // rows past M: zero scales (their codes are masked in the GEMM)
    for (int q = lane; q < NG; q += 64) sa_lds[q][wave] = 0.0f;
  }
  __syncthreads();

  // ---- the decode GEMM over this wave's runs, A from LDS
  const int64_t sw_row = (n0 + r) * NG;
  float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t rdw0 = 64 * r + 16 * ((0 + (j >> 1)) ^ ((r >> 2) & 3)) + 8 * (j & 1);
  const uint32_t rdw1 = 64 * r + 16 * ((2 + (j >> 1)) ^ ((r >> 2) & 3)) + 8 * (j & 1);
  const char* stw = reinterpret_cast<const char*>(&stage_w[wave][0][0]);
  for (int r0 = rbeg; r0 < rend; r0 += CR) {
    const int nr = rend - r0 < CR ? rend - r0 : CR;
    const int g0 = r0 * 128 / G;
    const int ng = (nr * 128 + G - 1) / G;
    if (r0 != rbeg) issue_w(r0, nr);
    scale_t swb[GPC];
#pragma unroll
    for (int u = 0; u < GPC; ++u) {
      const int uu = u < ng ? u : ng - 1;
      swb[u] = reinterpret_cast<const scale_t*>(g.sw)[sw_row + g0 + uu];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < GPC; ++u) {
      if (u >= ng) break;
      v4i acc = (v4i){0, 0, 0, 0};
      if (G == 32) {
        const int run = u >> 2, p = u & 3;
        const uint32_t ow = 1024u * run + 64u * r + 16u * (p ^ ((r >> 2) & 3)) + 4u * j;
        const uint32_t pw = *reinterpret_cast<const uint32_t*>(stw + ow);
        const uint32_t pa = arow ? *reinterpret_cast<const uint32_t*>(a_lds + fd_a_off(r0 + run, r, p) + 4 * j) : 0u;
        const uint2 av = make_uint2((pa << 4) & 0xF0F0F0F0u, pa & 0xF0F0F0F0u);
        const uint2 wv = make_uint2((pw << 4) & 0xF0F0F0F0u, pw & 0xF0F0F0F0u);
        acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, av),
                                                    __builtin_bit_cast(long, wv), acc, 0, 0, 0);
      }
#pragma unroll
      for (int m = u * MPG; G >= 64 && m < (u + 1) * MPG; ++m) {
        const int run = m >> 1, h = m & 1;
        const uint2 pw = *reinterpret_cast<const uint2*>(stw + 1024u * run + (h ? rdw1 : rdw0));
        uint2 pa = make_uint2(0u, 0u);
        if (arow)
          pa = *reinterpret_cast<const uint2*>(a_lds + fd_a_off(r0 + run, r, 2 * h + (j >> 1)) + 8 * (j & 1));
        v4i av, wv;
        av.x = (int)((pa.x << 4) & 0xF0F0F0F0u);
        av.y = (int)(pa.x & 0xF0F0F0F0u);
        av.z = (int)((pa.y << 4) & 0xF0F0F0F0u);
        av.w = (int)(pa.y & 0xF0F0F0F0u);
        wv.x = (int)((pw.x << 4) & 0xF0F0F0F0u);
        wv.y = (int)(pw.x & 0xF0F0F0F0u);
        wv.z = (int)((pw.y << 4) & 0xF0F0F0F0u);
        wv.w = (int)(pw.y & 0xF0F0F0F0u);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, wv, acc, 0, 0, 0);
      }
      // lane holds rows 4 j + v of column n0 + r; sums are 256x the true ones
      const float sw = (float)swb[u] * (1.0f / 256.0f);
      const float4 s4 = *reinterpret_cast<const float4*>(&sa_lds[g0 + u][4 * j]);
      const float sar[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) c[v] = fmaf((float)acc[v], sar[v] * sw, c[v]);
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][(4 * j + v) * 16 + r] = c[v];
  __syncthreads();
  if (tid < 256) {
    const int row = tid >> 4, col = tid & 15;
    if (row < g.M) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kFdWaves; ++w) s += part[w][tid];
      g.c[(int64_t)row * g.N + n0 + col] = s;
    }
  }
}

template <int G, bool F16>
static void launch_fd(const FusedDecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.N / 16));
  if (a.K == 4096)
    hipLaunchKernelGGL((rotate_quant_gemm_decode_kernel<G, F16, 2>), grid, dim3(kFdWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((rotate_quant_gemm_decode_kernel<G, F16, 1>), grid, dim3(kFdWaves * 64), 0, s, a);
}

template <int G>
static void launch_fd_g(const FusedDecodeArgs& a, hipStream_t s) {
  if (a.scale_f16) launch_fd<G, true>(a, s); else launch_fd<G, false>(a, s);
}

hipError_t launch_rotate_quant_gemm_decode(const FusedDecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 32: launch_fd_g<32>(a, s); break;
    case 64: launch_fd_g<64>(a, s); break;
    case 128: launch_fd_g<128>(a, s); break;
    default: launch_fd_g<256>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace hr
