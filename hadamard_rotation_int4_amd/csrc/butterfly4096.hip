// HARP-style butterfly for n = 4096: 12 stages of 2x2 blocks on pairs at
// stride 2^s, then the gather permutation; optional fused int4 quantization.
//
// Source: HARP abstract (a rotation as a product of sparse butterfly-like
// block-orthogonal stages) and HARP technical summary (gist.science), sections
// 2.1 (stride stages), 2.2 (block kernel Q(theta) G_2) and 2.4 (O(d log d)
// application without materialised permutations).
//
// One workgroup of 512 threads per row, persistent over rows.  With an fp32
// output, input rows stream through a ring of kBfRing LDS stages filled by
// global_load_lds (kBfRing rows in flight per CU without holding registers):
// wave w loads bytes 2048 w .. 2048 w + 2047 of a row, which are exactly the
// 8-element slices of its own 64 threads, so a wave waits only for its own
// loads.  With codes only, the next two rows are prefetched into registers.  Each
// thread owns 8 elements of the row per pass; the 12 stages run as 4 passes of 3
// register stages.  In pass k the thread's 8 registers are the elements whose
// index bits 3k..3k+2 take all 8 values, the other 9 bits being the thread
// index; between passes the row goes through LDS.  Because a thread owns the
// same pairs in every row, its 12 x 4 pairs' coefficients stay in registers
// for the kernel's lifetime.  Passes 1 and 2 exchange elements only within a
// wave, so of the four exchanges per row only pass 3 and the permutation take
// a workgroup barrier.  The LDS index is padded by 8 floats every 64
// (p = i + 8 * (i >> 6)) so that the one strided pass (k = 1) is bank-conflict
// free; the other passes access consecutive elements.
#include "hr_internal.h"
#include "fwht2048.h"

namespace hr {

constexpr int kBfN = 4096;
constexpr int kBfThreads4096 = 512;
constexpr int kBfLds = kBfN + 8 * (kBfN / 64);
constexpr int kBfRing = 3;

// Workgroup barrier for the LDS transposes: this wave's LDS accesses are
// complete (lgkmcnt 0) before it arrives.  Unlike __syncthreads it does not
// also wait for the ring's loads still in flight (vmcnt), which would drain
// the prefetch at every transpose; the memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bf_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void bf_lds_load16(const void* gp, void* lp) {
  // nontemporal: the rows are read once (fp32 32768 x 4096, same box: 213.6
  // -> 208.0-210.5 us with fp32 output, 174-176 -> 172.6-174 us codes only)
  __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 2);
}

__device__ __forceinline__ int bf_pad(int i) { return i + 8 * (i >> 6); }

// element index of register r of thread t in pass k: bits 3k..3k+2 = r
__device__ __forceinline__ int bf_idx(int t, int k, int r) {
  const int lo = t & ((1 << (3 * k)) - 1);
  const int hi = t >> (3 * k);
  return lo | (r << (3 * k)) | (hi << (3 * k + 3));
}

// register holding the lower element of pair q (0..3) of the stage on
// register bit b
__device__ __forceinline__ constexpr int bf_r0(int q, int b) {
  return ((q >> b) << (b + 1)) | (q & ((1 << b) - 1));
}

template <bool PRECOND, bool TRANSPOSE>
__device__ __forceinline__ void bf_block(float& a, float& b, float2 k) {
  const float u = a, v = b;
  if (PRECOND) {                 // [[k.x, k.y], [k.y, -k.x]] (symmetric)
    a = fmaf(k.x, u, k.y * v);
    b = fmaf(k.y, u, -k.x * v);
  } else if (!TRANSPOSE) {       // [[c, -s], [s, c]]
    a = fmaf(k.x, u, -k.y * v);
    b = fmaf(k.y, u, k.x * v);
  } else {                       // [[c, s], [-s, c]]
    a = fmaf(k.x, u, k.y * v);
    b = fmaf(-k.y, u, k.x * v);
  }
}

template <bool PRECOND, bool TRANSPOSE>
__device__ __forceinline__ void bf_stage(float (&v)[8], const float2 (&cf)[4], int b) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = bf_r0(q, b);
    bf_block<PRECOND, TRANSPOSE>(v[r0], v[r0 | (1 << b)], cf[q]);
  }
}

template <bool PRECOND, bool INVERSE, bool OUT_Y, int G, bool SCALE_F16>
__global__ __launch_bounds__(kBfThreads4096, 1) void butterfly4096_kernel(
    const float* __restrict__ x, float* __restrict__ y, int64_t rows,
    const float2* __restrict__ coeffs, const int* __restrict__ perm,
    uint8_t* __restrict__ codes, void* __restrict__ scales) {
  constexpr int N = kBfN, HALF = N / 2;
  __shared__ __attribute__((aligned(16))) float lds[3][kBfLds];
  // the ring only where the row's fp32 output makes the kernel memory-bound;
  // with codes only, its extra LDS traffic costs more than it hides
  constexpr bool RING = OUT_Y;
  __shared__ __attribute__((aligned(16))) float ring[RING ? kBfRing : 1][RING ? N : 4];
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;

  // per-thread coefficients of its 4 pairs in each of the 12 stages
  float2 cf[12][4];
#pragma unroll
  for (int s = 0; s < 12; ++s) {
    const int k = s / 3, b = s % 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = bf_idx(t, k, bf_r0(q, b));
      const int p = ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
      cf[s][q] = coeffs[s * HALF + p];
    }
  }
  int pm[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pm[r] = perm ? perm[8 * t + r] : 8 * t + r;

  // row r goes to ring stage: wave wv's two loads put bytes 2048 wv + 16 lane
  // (+ 1024) of the row at the same offsets of the stage
  auto issue = [&](int64_t r, int st) {
    const char* src = reinterpret_cast<const char*>(x + r * N) + 2048 * wv + 16 * lane;
    char* dst = reinterpret_cast<char*>(&ring[st][0]) + 2048 * wv;
    bf_lds_load16(src, dst);
    bf_lds_load16(src + 1024, dst + 1024);
  };
  const int64_t step = gridDim.x;
  if (RING) {
#pragma unroll
    for (int i = 0; i < kBfRing; ++i)
      if ((int64_t)blockIdx.x + i * step < rows) issue((int64_t)blockIdx.x + i * step, i);
  }
  // thread t's elements 8t .. 8t+7: bytes 32 t of the stage
  const uint32_t rd_off = 32u * (uint32_t)t;

  // the row's transform, gather and outputs, from the thread's 8 elements v
  auto body = [&](int64_t row, float (&v)[8]) {
    if (!INVERSE) {
      // pass 0: stages 0, 1, 2 on elements 8t .. 8t+7
#pragma unroll
      for (int b = 0; b < 3; ++b) bf_stage<PRECOND, false>(v, cf[b], b);
      // Passes 1 and 2 move elements only within a wave (wave w writes and
      // reads elements 512 w .. 512 w + 511), and a wave's LDS accesses take
      // effect in issue order, so they need no workgroup barrier.  Pass 3 and
      // the gather cross waves.  Buffers: passes 1 and 3 in 0, pass 2 in 1,
      // the gather in 2, so that every access by one wave to a region another
      // wave used is separated by one of the two barriers.
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        float* bk = lds[k == 2 ? 1 : 0];
#pragma unroll
        for (int r = 0; r < 8; ++r) bk[bf_pad(bf_idx(t, k - 1, r))] = v[r];
        if (k < 3) asm volatile("" ::: "memory");    // keep the reads after the writes
        else bf_barrier();
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = bk[bf_pad(bf_idx(t, k, r))];
#pragma unroll
        for (int b = 0; b < 3; ++b) bf_stage<PRECOND, false>(v, cf[3 * k + b], b);
      }
      // gather: out[8t + r] = z[perm[8t + r]]
      float* bg = lds[2];
#pragma unroll
      for (int r = 0; r < 8; ++r) bg[bf_pad(bf_idx(t, 3, r))] = v[r];
      bf_barrier();
      if (perm) {
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = bg[bf_pad(pm[r])];
      } else {
        // identity: elements 8t .. 8t+7 are 8 consecutive padded slots, read
        // as two 16-byte loads (eight scalar loads at a stride of 8 conflict)
        const f32x4* src = reinterpret_cast<const f32x4*>(&bg[bf_pad(8 * t)]);
        const f32x4 u0 = src[0], u1 = src[1];
        v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
        v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
      }
    } else {
      // scatter z[perm[i]] = x[i], then the transposed stages in reverse
      // order.  As in the forward direction only the scatter and the pass-3
      // exchange cross waves: the scatter goes to buffer 2, pass 3 writes
      // buffer 0, pass 2 buffer 1 and pass 1 buffer 0 again, with workgroup
      // barriers after the first two only.
      float* bs = lds[2];
      if (perm) {
#pragma unroll
        for (int r = 0; r < 8; ++r) bs[bf_pad(pm[r])] = v[r];
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(&bs[bf_pad(8 * t)]);
        dst[0] = (f32x4){v[0], v[1], v[2], v[3]};
        dst[1] = (f32x4){v[4], v[5], v[6], v[7]};
      }
      bf_barrier();
      float* src = bs;
#pragma unroll
      for (int k = 3; k >= 1; --k) {
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = src[bf_pad(bf_idx(t, k, r))];
#pragma unroll
        for (int b = 2; b >= 0; --b) bf_stage<PRECOND, true>(v, cf[3 * k + b], b);
        float* dstb = lds[k == 2 ? 1 : 0];
#pragma unroll
        for (int r = 0; r < 8; ++r) dstb[bf_pad(bf_idx(t, k, r))] = v[r];
        if (k == 3) bf_barrier();
        else asm volatile("" ::: "memory");      // keep the reads after the writes
        src = dstb;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = src[bf_pad(bf_idx(t, 0, r))];
#pragma unroll
      for (int b = 2; b >= 0; --b) bf_stage<PRECOND, true>(v, cf[b], b);
    }
    // thread t now holds output elements 8t .. 8t+7
    if (OUT_Y) {
      f32x4* yr = reinterpret_cast<f32x4*>(y + row * N) + 2 * t;
      __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, yr);
      __builtin_nontemporal_store((f32x4){v[4], v[5], v[6], v[7]}, yr + 1);
    }
    if (G > 0) {
      // group of G = G/8 consecutive lanes x 8 registers
      float a = fmaxf(fabsf(v[0]), fabsf(v[1]));
#pragma unroll
      for (int r = 2; r < 8; ++r) a = fmaxf(a, fabsf(v[r]));
      uint32_t ab = __float_as_uint(a);
      ab = umax_dpp<kQuadXor1>(ab);
      ab = umax_dpp<kQuadXor2>(ab);
      if (G >= 64) ab = umax_dpp<kRowHalfMirror>(ab);
      if (G >= 128) ab = umax_dpp<kRowMirror>(ab);
      if (G >= 256) {
        const uint32_t o = (uint32_t)__shfl_xor((int)ab, 16, 64);
        ab = ab > o ? ab : o;
      }
      const float s32 = div7(__uint_as_float(ab));
      const float s = SCALE_F16 ? (float)(_Float16)s32 : s32;
      // an fp32 scale below 2^-100 would overflow its reciprocal: the group's
      // values and scale are then both taken x 2^64 (exact; same quotients)
      const float up = (!SCALE_F16 && s < 0x1p-100f) ? 0x1p64f : 1.0f;
      const float k = s > 0.0f ? __builtin_amdgcn_rcpf(s * up) : 0.0f;
      const bool need_clamp = s > 0.0f && s < (SCALE_F16 ? 6.103515625e-05f : 1.17549435e-38f);
      const bool clamp = __builtin_amdgcn_ballot_w64(need_clamp) != 0;
      const float M = 12582920.0f;              // 1.5 * 2^23 + 8
      float r8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) r8[r] = fmaf(SCALE_F16 ? v[r] : v[r] * up, k, M);
      if (clamp) {
#pragma unroll
        for (int r = 0; r < 8; ++r) r8[r] = __builtin_amdgcn_fmed3f(r8[r], M - 7.0f, M + 7.0f);
      }
      __builtin_nontemporal_store(pack8(r8), reinterpret_cast<uint32_t*>(codes + row * (N / 2)) + t);
      if ((t & (G / 8 - 1)) == 0) {
        const int64_t si = row * (N / G) + (8 * t) / G;
        if (SCALE_F16) reinterpret_cast<_Float16*>(scales)[si] = (_Float16)s32;
        else reinterpret_cast<float*>(scales)[si] = s32;
      }
    }
  };

  if (RING) {
    int st = 0, iter = 0;
    for (int64_t row = blockIdx.x; row < rows; row += step, st = st + 1 == kBfRing ? 0 : st + 1, ++iter) {
      float v[8];
      // wait for this row's two loads.  Vector memory operations complete in
      // issue order; the ones issued after them are the younger rows' loads (two
      // each) and the stores of the rows processed since: SU per row, two fp32
      // stores and the code and scale stores.  Every wave issues each of them
      // (a wave's 64 threads always include scale-storing ones, since G / 8 <= 32),
      // so the count is exact.  Near the end of the rows everything is drained.
      f32x4 n0, n1;
      const uint32_t addr = (uint32_t)(uintptr_t)&ring[st][0] + rd_off;
      constexpr int SU = (OUT_Y ? 2 : 0) + (G > 0 ? 2 : 0);
#define HR_BFR(N)                                                                            \
      asm volatile("s_waitcnt vmcnt(" #N ")\n\tds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\t" \
                   "s_waitcnt lgkmcnt(0)"                                                     \
                   : "=v"(n0), "=v"(n1)                                                       \
                   : "v"(addr)                                                                \
                   : "memory")
      static_assert(kBfRing == 3, "the wait counts below assume three ring stages");
      if (row + (kBfRing - 1) * step < rows) {
        const int done = iter < kBfRing ? iter : kBfRing;   // rows processed whose stores are younger
        static_assert(SU == 2 || SU == 4, "fp32 out, codes, or both");
        if (done == 0) HR_BFR(4);
        else if (SU == 2) { if (done == 1) HR_BFR(6); else if (done == 2) HR_BFR(8); else HR_BFR(10); }
        else { if (done == 1) HR_BFR(8); else if (done == 2) HR_BFR(12); else HR_BFR(16); }
      } else {
        HR_BFR(0);
      }
#undef HR_BFR
      v[0] = n0.x; v[1] = n0.y; v[2] = n0.z; v[3] = n0.w;
      v[4] = n1.x; v[5] = n1.y; v[6] = n1.z; v[7] = n1.w;
      if (row + kBfRing * step < rows) issue(row + kBfRing * step, st);
      body(row, v);
    }
  } else {
    // register prefetch two rows deep, in two register sets used in turn (a
    // copy from one set to the other would wait for the younger load).  The
    // loads are unconditional: past the last row a set reloads a row already
    // held (never used), so that no register merges loaded and unloaded values
    auto load = [&](int64_t r, f32x4& q0, f32x4& q1) {
      const f32x4* xr = reinterpret_cast<const f32x4*>(x + r * N) + 2 * t;
      q0 = __builtin_nontemporal_load(xr);
      q1 = __builtin_nontemporal_load(xr + 1);
    };
    auto take = [&](const f32x4& q0, const f32x4& q1, float (&v)[8]) {
      v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
      v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    };
    const int64_t r0 = blockIdx.x;
    if (r0 < rows) {
      f32x4 a0, a1, b0, b1;
      load(r0, a0, a1);
      load(r0 + step < rows ? r0 + step : r0, b0, b1);
      for (int64_t row = r0; row < rows; row += 2 * step) {
        float v[8];
        take(a0, a1, v);
        load(row + 2 * step < rows ? row + 2 * step : row, a0, a1);
        body(row, v);
        if (row + step >= rows) break;
        float w[8];
        take(b0, b1, w);
        load(row + 3 * step < rows ? row + 3 * step : row, b0, b1);
        body(row + step, w);
      }
    }
  }
}

template <bool PRECOND, bool INVERSE, bool OUT_Y, int G, bool F16>
static void bf_launch(const ButterflyArgs& a, hipStream_t s) {
  const int64_t blocks = a.rows < 256 ? a.rows : 256;
  hipLaunchKernelGGL((butterfly4096_kernel<PRECOND, INVERSE, OUT_Y, G, F16>), dim3((unsigned)blocks),
                     dim3(kBfThreads4096), 0, s, a.x, a.y, a.rows,
                     reinterpret_cast<const float2*>(a.coeffs), a.perm, a.codes, a.scales);
}

template <bool PRECOND>
static bool bf_dispatch(const ButterflyArgs& a, hipStream_t s) {
  if (a.inverse) {
    if (a.codes || !a.y) return false;
    bf_launch<PRECOND, true, true, 0, false>(a, s);
    return true;
  }
  if (!a.codes) {
    bf_launch<PRECOND, false, true, 0, false>(a, s);
    return true;
  }
#define HR_BFQ(G)                                                                     \
  case G:                                                                             \
    if (a.y) {                                                                        \
      if (a.scale_f16) bf_launch<PRECOND, false, true, G, true>(a, s);                \
      else bf_launch<PRECOND, false, true, G, false>(a, s);                           \
    } else {                                                                          \
      if (a.scale_f16) bf_launch<PRECOND, false, false, G, true>(a, s);               \
      else bf_launch<PRECOND, false, false, G, false>(a, s);                          \
    }                                                                                 \
    return true;
  switch (a.group) {
    HR_BFQ(32)
    HR_BFQ(64)
    HR_BFQ(128)
    HR_BFQ(256)
    default: return false;
  }
#undef HR_BFQ
}

// Handles n == 4096; returns false for other sizes (general kernel).
bool launch_butterfly4096(const ButterflyArgs& a, hipStream_t s) {
  if (a.n != kBfN) return false;
  return a.precondition ? bf_dispatch<true>(a, s) : bf_dispatch<false>(a, s);
}

}  // namespace hr
