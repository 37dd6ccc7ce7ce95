// W4A4 and W4A8 GEMMs on CDNA4 int8 MFMA, tiled kernels.
//
// What is computed ("Experiment -- Hadamard rotation for int4 (W4A4)
// accuracy", Hypothesis and Verdict; W4A8 is the same page's act8/wt4 rows of
// Results): C = A W^T with
//   acc[m][n][g] = sum_{k in group g} a[m][k] w[n][k]   (exact int32)
//   C[m][n]      = sum_g sA[m][g] sW[n][g] acc[m][n][g]  (fp32)
//
// Operand preparation.  A packed byte holds codes (k, k+1) in its (low, high)
// nibble.  x & 0xF0F0F0F0 turns a dword of 8 codes into 4 int8 bytes equal to
// 16 * (odd codes), (x << 4) & 0xF0F0F0F0 into 16 * (even codes).  Both
// operands get the same K permutation, so every int32 sum is exactly 256 times
// the true group sum; the 1/256 is applied (exactly) to the fp32 result.  In
// W4A8 the activations are int8 codes already: v_perm_b32 puts their bytes in
// the order the weight unpack produces (k = 0 2 4 6 | 1 3 5 7 per 8 codes),
// and the sums are 16 times the true ones.
//
// Prefill kernel (M > 16): a 128x128 output tile per workgroup of 4 waves,
// 64x64 per wave as 2x2 v_mfma_i32_32x32x32_i8 tiles, stages of up to 128
// codes unpacked once into LDS; the per-group scale fusion is described at
// the kernel.  Measured on MI355X, vector-ALU work of one wave does not run
// alongside the MFMAs of another wave on the same SIMD, while independent
// vector instructions that follow a wave's own MFMA do; the kernel therefore
// interleaves each wave's epilogue with its own MFMAs.
//
// Decode kernel (M <= 16): one 16x16 output tile per workgroup of 16 waves
// that split K; operands are staged through LDS by global_load_lds, the
// partial tiles are summed through LDS.
#include <type_traits>

#include "hr_internal.h"
#include "hr_device.h"

namespace hr {

typedef int v4i __attribute__((ext_vector_type(4)));

// 16 int8 codes in natural order -> the K order of unpack16 (k = 0 2 4 6,
// 1 3 5 7, 8 10 12 14, 9 11 13 15)
__device__ __forceinline__ v4i order_int8(uint4 p) {
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(p.y, p.x, 0x06040200u);
  r.y = (int)__builtin_amdgcn_perm(p.y, p.x, 0x07050301u);
  r.z = (int)__builtin_amdgcn_perm(p.w, p.z, 0x06040200u);
  r.w = (int)__builtin_amdgcn_perm(p.w, p.z, 0x07050301u);
  return r;
}

__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  r.x = (int)((p.x << 4) & 0xF0F0F0F0u);
  r.y = (int)(p.x & 0xF0F0F0F0u);
  r.z = (int)((p.y << 4) & 0xF0F0F0F0u);
  r.w = (int)(p.y & 0xF0F0F0F0u);
  return r;
}

template <bool F16>
__device__ __forceinline__ float ld_scale(const void* p, int64_t idx) {
  return F16 ? (float)reinterpret_cast<const _Float16*>(p)[idx]
             : reinterpret_cast<const float*>(p)[idx];
}

constexpr int kBM = 128, kBN = 128;

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// XOR applied to the row index of chunk pair q (chunks 2q, 2q + 1) in the
// LDS operand buffers, laid out [chunk][128 rows] of 16-byte slots.  A
// 16-byte store phase covers 8 or 16 lanes: rows r0 .. r0 + 16/PPR - 1 (or
// half of them) times the PPR pieces of a row (PPR packed 16-byte pieces per
// row and stage), writing chunk 2p (or 2p + 1) of piece p.  With the
// constants {0, 6, 10, 12} (PPR = 4) or {0, 12} (PPR = 2) those writes hit
// 16-byte bank groups that differ modulo 8 and modulo 16.  A read phase
// takes one chunk of 8 or 16 consecutive rows, which an XOR below 16 only
// permutes.  Both patterns are free of bank conflicts.
template <int PPR>
__device__ __forceinline__ constexpr int row_xor(int q) {
  return PPR == 4 ? (q == 0 ? 0 : q == 1 ? 6 : q == 2 ? 10 : 12) : (q == 0 ? 0 : 12);
}

// XOR applied to the row index of int8 A chunk c (PPA = 16-byte A pieces per
// row and stage, one chunk each).  A store phase covers one row (8 lanes,
// PPA = 8) or two rows (PPA = 4) times the PPA chunks, or twice that for 16
// lanes; its 16-byte bank groups must differ modulo 8 (8 lanes) and modulo 16
// (16 lanes).  2c + (c >> 2) = {0, 2, 4, 6, 9, 11, 13, 15} (PPA = 8) and
// 4c + 2 (c >> 1) = {0, 4, 10, 14} (PPA = 4) do both; reads take one chunk of
// 8 or 16 consecutive rows, which an XOR below 16 only permutes.
template <int PPA>
__device__ __forceinline__ constexpr int a8_xor(int c) {
  return PPA == 8 ? 2 * c + (c >> 2) : 4 * c + 2 * (c >> 1);
}

template <int V>
struct IntC { static constexpr int value = V; };

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x2, kSchedMfma = 0x8, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// Prefill kernel.  A 128x128 output tile per workgroup of 4 waves, 64x64 per
// wave as 2x2 tiles of v_mfma_i32_32x32x32_i8.  Per pipeline stage of KS
// codes: every thread buffer-loads 16-byte pieces of packed rows (PPR lanes
// cover the bytes a row holds for a stage), unpacks them once and stores them
// to LDS in operand order; the waves read their fragments with one
// ds_read_b128 per 32-row block and K-step.  Lane l of a fragment holds row
// l % 32 and chunk 2s + l / 32 of K-step s, i.e. codes 32 s .. 32 s + 31 of
// the stage, in the same (permuted) order for both operands.
//
// Group epilogue with fp16 scales: the outer product sA (x) sW of the group
// is itself one v_mfma_f32_32x32x16_f16 per 32x32 tile (lane l < 32 puts the
// scale of row / column l in K slot 0, every other slot is zero; products of
// two fp16 values are exact in fp32), so the vector ALU only converts the
// int32 sums and runs one fma per output and group.  With fp32 scales the
// product sA * sW is formed on the vector ALU.
//
// Overlap: each stage runs in two halves.  The first half issues the MFMAs
// of the upper tiles (i = 0) while the vector ALU finishes the previous
// group of the lower tiles (i = 1); the second half issues the lower tiles'
// MFMAs while the upper tiles' group is converted and accumulated.  Every
// tile's sums are consumed before its next group overwrites them, so no
// second accumulator set is needed.  Group scales go through a 3-deep LDS
// ring, so the lower tiles can still read the previous group's scales after
// other waves have stored the next stage's.  Stages are unrolled in pairs so
// that the LDS buffer of every access is a compile-time offset.
template <int G, bool F16, bool WRITE_ACC, bool A8>
__global__ __launch_bounds__(256, 2) void w4a4_gemm_tile_kernel(GemmArgs g) {
  constexpr int KS = G < 128 ? G : 128;   // codes per pipeline stage
  constexpr int STEPS = KS / 32;          // MFMA K-steps per stage
  constexpr int SPG = G / KS;             // stages per group (1 or 2)
  constexpr int PPR = KS / 32;            // 16-byte packed pieces per row and stage
  constexpr int PPA = A8 ? 2 * PPR : PPR; // 16-byte pieces per A row and stage
  constexpr int LPO = PPR / 2;            // W pieces per thread and stage
  constexpr int LPA = PPA / 2;            // A pieces per thread and stage
  constexpr int LOADS = LPA + LPO;
  constexpr int OPB = (KS / 16) * 128 * 16;   // bytes of one operand stage in LDS
  constexpr int LSC = 4 * OPB;            // byte offset of the scale ring
  constexpr int SB = F16 ? 2 : 4;         // bytes per scale
  __shared__ __attribute__((aligned(16))) char smem[4 * OPB + 3 * 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const uint32_t hmask = h ? 0u : 0xFFFFFFFFu;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t rowb = g.K / 2;           // bytes per packed row
  const int64_t rowb_a = A8 ? g.K : rowb; // bytes per A row
  const int ngroups = (int)(g.K / G);
  const int nstages = (int)(g.K / KS);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // Operand panels and this thread's pieces: A piece t < LPA is tile row
  // srow_a + t * 256 / PPA, 16-byte piece spc_a; W piece LPA + t is row
  // srow + t * 256 / PPR, piece spc.  A rows past M read row 0 of the panel
  // instead (a valid address; never stored).
  const __amdgpu_buffer_rsrc_t rs_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)(g.a + m0 * rowb_a), 0, (int)(128 * rowb_a), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_w =
      __builtin_amdgcn_make_buffer_rsrc((void*)(g.w + n0 * rowb), 0, (int)(128 * rowb), 0x00020000);
  const int srow = tid / PPR, spc = tid % PPR;
  const int srow_a = tid / PPA, spc_a = tid % PPA;
  int voff[LOADS];
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    if (t < LPA) {
      const int r = srow_a + t * (256 / PPA);
      voff[t] = (m0 + r >= g.M ? 0 : r) * (int)rowb_a + 16 * spc_a;
    } else {
      voff[t] = (srow + (t - LPA) * (256 / PPR)) * (int)rowb + 16 * spc;
    }
  }
  // scale row of this thread: threads 0-127 (waves 0, 1) A rows, 128-255 W rows
  const int64_t sr = tid < kBM ? (m0 + tid < g.M ? m0 + tid : m0) : n0 + tid - kBM;
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wave < 2 ? g.sa : g.sw), 0, 0x7FFFFFFF, 0x00020000);
  const int svoff = (int)(sr * ngroups * SB);

  // LDS byte offsets: this thread's store slot (chunk 2 spc, row srow), and
  // the fragment read slots of K-step ks (chunk 2 ks + h, row wm + l32 or
  // wn + l32) within an operand stage.  int8 A pieces are one chunk each
  // (chunk spc_a), rows XORed with a8_xor<PPA>(chunk).
  const int st_off = (2 * spc * 128 + (srow ^ row_xor<PPR>(spc))) * 16;
  const int st_off_a = (spc_a * 128 + (srow_a ^ a8_xor<PPA>(spc_a))) * 16;
  int rd_a[STEPS], rd_b[STEPS];
#pragma unroll
  for (int ks = 0; ks < STEPS; ++ks) {
    const int xa = A8 ? a8_xor<PPA>(2 * ks + h) : row_xor<PPR>(ks);
    rd_a[ks] = (h * 128 + wm + (l32 ^ xa)) * 16;
    rd_b[ks] = OPB + (h * 128 + wn + (l32 ^ row_xor<PPR>(ks))) * 16;
  }

  v16f c[2][2];
  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      c[i][j] = (v16f){};
      acc[i][j] = (v16i){};
    }

  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u pre[LOADS];
  uint32_t psc = 0;
  auto load_stage = [&](int s) {
    const int so = s * (KS / 2), so_a = A8 ? s * KS : so;
#pragma unroll
    for (int t = 0; t < LOADS; ++t)
      pre[t] = __builtin_amdgcn_raw_buffer_load_b128(t < LPA ? rs_a : rs_w, voff[t],
                                                     t < LPA ? so_a : so, 0);
    const int gso = (s / SPG) * SB;
    psc = F16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs_s, svoff, gso, 0)
              : __builtin_amdgcn_raw_buffer_load_b32(rs_s, svoff, gso, 0);
  };
  auto store_stage = [&](auto bufc, int ring) {
    char* sb = smem + decltype(bufc)::value * 2 * OPB;
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      if (A8 && t < LPA) {
        char* d = sb + t * (256 / PPA) * 16 + st_off_a;
        *reinterpret_cast<v4i*>(d) = order_int8(make_uint4(pre[t].x, pre[t].y, pre[t].z, pre[t].w));
        continue;
      }
      const int op = t < LPA ? 0 : 1, tt = t < LPA ? t : t - LPA;
      char* d = sb + op * OPB + tt * (256 / PPR) * 16 + st_off;
      *reinterpret_cast<v4i*>(d) = unpack16(make_uint2(pre[t].x, pre[t].y));
      *reinterpret_cast<v4i*>(d + 2048) = unpack16(make_uint2(pre[t].z, pre[t].w));
    }
    *reinterpret_cast<uint32_t*>(smem + LSC + ring * 1024 + tid * 4) = psc;
  };

  // MFMAs of tiles (i, 0) and (i, 1) over one stage; the B fragments are read
  // in the first half and kept for the second
  auto mfma_half = [&](auto bufc, int i, bool zero_first, v4i (&bfr)[STEPS][2], bool read_b) {
    const char* sb = smem + decltype(bufc)::value * 2 * OPB;
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks) {
      const v4i af = *reinterpret_cast<const v4i*>(sb + rd_a[ks] + (2 * ks * 128 + 32 * i) * 16);
      if (read_b) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[ks][j] = *reinterpret_cast<const v4i*>(sb + rd_b[ks] + (2 * ks * 128 + 32 * j) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = (zero_first && ks == 0)
                        ? __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bfr[ks][j], (v16i){}, 0, 0, 0)
                        : __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bfr[ks][j], acc[i][j], 0, 0, 0);
    }
  };
  // group epilogue of tiles (i, 0) and (i, 1) with the scales in ring slot
  // ring; lane holds acc[i][j][v] of row wm + 32 i + 8 (v / 4) + 4 h + v % 4,
  // column wn + 32 j + l32
  auto epilogue = [&](int i, int ring, int gi) {
    const char* ls = smem + LSC + ring * 1024;
    if (F16) {
      const uint32_t ra = *reinterpret_cast<const uint32_t*>(ls + (wm + 32 * i + l32) * 4) & hmask;
      const v4h sa = __builtin_bit_cast(v4h, (v2i){(int)ra, 0});
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t rw = *reinterpret_cast<const uint32_t*>(ls + (kBM + wn + 32 * j + l32) * 4) & hmask;
        const v4h sw = __builtin_bit_cast(v4h, (v2i){(int)rw, 0});
        const v16f p = __builtin_amdgcn_mfma_f32_32x32x8f16(sa, sw, (v16f){}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = fmaf((float)acc[i][j][v], p[v], c[i][j][v]);
      }
    } else {
      float sa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(ls + (wm + 32 * i + 8 * q + 4 * h) * 4);
        sa[4 * q] = __uint_as_float(t4.x);
        sa[4 * q + 1] = __uint_as_float(t4.y);
        sa[4 * q + 2] = __uint_as_float(t4.z);
        sa[4 * q + 3] = __uint_as_float(t4.w);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sw = *reinterpret_cast<const float*>(ls + (kBM + wn + 32 * j + l32) * 4);
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = fmaf((float)acc[i][j][v], sa[v] * sw, c[i][j][v]);
      }
    }
    if (WRITE_ACC && gi >= 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const int64_t col = n0 + wn + 32 * j + l32;
          if (row < g.M) g.group_acc[(row * g.N + col) * ngroups + gi] = acc[i][j][v] >> (A8 ? 4 : 8);
        }
    }
  };

  // one pipeline stage; the stage's LDS buffer (s & 1) is the template
  // constant, and with two stages per group so is its position in the group
  auto stage = [&](int s, auto bufc) {
    constexpr int B = decltype(bufc)::value;
    constexpr int SUB = SPG == 1 ? 0 : B;
    const int gi = s / SPG;
    const int ring = s % 3;
    // the last stage reloads itself (a valid address; the copy is never read)
    load_stage(s + 1 < nstages ? s + 1 : s);
    v4i bfr[STEPS][2];
    // first half: fragment and scale reads, then each MFMA followed by a run
    // of the lower tiles' epilogue on the vector ALU
    mfma_half(bufc, 0, SUB == 0, bfr, true);
    if (SUB == 0) epilogue(1, ring == 0 ? 2 : ring - 1, gi - 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 16, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // second half: the lower tiles' MFMAs, the upper tiles' epilogue and the
    // next stage's unpack and LDS stores
    mfma_half(bufc, 1, SUB == 0, bfr, false);
    if (SUB == SPG - 1) epilogue(0, ring, gi);
    store_stage(IntC<B ^ 1>{}, ring == 2 ? 0 : ring + 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 12, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  // ring slot 2 stands for the group before the first one: zero scales make
  // the lower tiles' first (empty) epilogue add nothing
  *reinterpret_cast<uint32_t*>(smem + LSC + 2 * 1024 + tid * 4) = 0u;
  load_stage(0);
  store_stage(IntC<0>{}, 0);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= nstages; s += 2) {
    stage(s, IntC<0>{});
    stage(s + 1, IntC<1>{});
  }
  if (s < nstages) stage(s, IntC<0>{});
  epilogue(1, (nstages - 1) % 3, ngroups - 1);

  // every int32 sum is 256 (W4A8: 16) times the true one: each int4 operand
  // carries 16 x code
  constexpr float kUnscale = A8 ? 1.0f / 16.0f : 1.0f / 256.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < g.M) {
#pragma unroll
        for (int j = 0; j < 2; ++j) g.c[row * g.N + n0 + wn + 32 * j + l32] = c[i][j][v] * kUnscale;
      }
    }
}


__device__ __forceinline__ void gemm_lds_load16(const void* gp, void* lp) {
  __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}

// W8A8 prefill kernel (M > 16): both operands one int8 code per element (the
// W4A4 GEMM with its codes held in int8, or W8A8).  Tiling, waves, MFMAs, the
// group epilogue and the scale ring are those of the packed kernel above;
// the operands need no unpacking, so each stage's 16-byte pieces go from
// memory straight into LDS with global_load_lds, without registers or vector
// instructions.  LDS layout of one operand stage: tile row r keeps its SPR =
// KS / 16 pieces at slots r SPR + (c ^ f(r)), f(r) = (r / (16 / SPR)) % SPR.
// A load instruction fills 64 consecutive slots, i.e. whole rows read as
// contiguous runs of KS bytes; the 16 lanes of a fragment-read phase (16
// consecutive rows, one piece c) hit 16 different bank groups.  Codes are
// used as they are: the int32 sums are the true group sums.
template <int G, bool F16, bool WRITE_ACC>
__global__ __launch_bounds__(256, 2) void w8a8_gemm_tile_kernel(GemmArgs g) {
  constexpr int KS = G < 128 ? G : 128;   // codes per row and stage
  constexpr int STEPS = KS / 32;          // MFMA K-steps per stage
  constexpr int SPG = G / KS;             // stages per group (1 or 2)
  constexpr int SPR = KS / 16;            // 16-byte pieces per row and stage
  constexpr int RPF = 16 / SPR;           // f(r) = (r / RPF) % SPR
  constexpr int OPB = 128 * KS;           // bytes of one operand stage
  constexpr int LSC = 4 * OPB;            // byte offset of the scale ring
  constexpr int SB = F16 ? 2 : 4;         // bytes per scale
  constexpr int NDMA = 2 * 128 * SPR / 64;   // load instructions per stage
  constexpr int DPW = NDMA / 4;              // ... per wave
  __shared__ __attribute__((aligned(16))) char smem[4 * OPB + 3 * 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const uint32_t hmask = h ? 0u : 0xFFFFFFFFu;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t K = g.K;
  const int ngroups = (int)(K / G);
  const int nstages = (int)(K / KS);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // this lane's source of load instruction j (slot block q = DPW wave + j of
  // the stage: operand q / (NDMA / 2), its 64 slots from 64 (q % (NDMA / 2)));
  // A rows past M read row 0 of the panel instead (a valid address, never
  // stored).  Per stage the source advances by KS bytes.
  // (32-bit offsets from the two panels' first rows keep the registers low)
  const int8_t* pa = reinterpret_cast<const int8_t*>(g.a) + m0 * K;
  const int8_t* pw = reinterpret_cast<const int8_t*>(g.w) + n0 * K;
  int off[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int q = DPW * wave + j;
    const int op = q / (NDMA / 2), sl = 64 * (q % (NDMA / 2)) + lane;
    const int r = sl / SPR, c = (sl % SPR) ^ ((r / RPF) % SPR);
    const int rr = op == 0 && m0 + r >= g.M ? 0 : r;
    off[j] = rr * (int)K + 16 * c;
  }
  auto issue = [&](int s, int buf) {
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int q = DPW * wave + j;
      const int op = q / (NDMA / 2);
      gemm_lds_load16((op == 0 ? pa : pw) + off[j] + s * KS,
                      smem + buf * 2 * OPB + op * OPB + 64 * 16 * (q % (NDMA / 2)));
    }
  };
  // scale row of this thread: threads 0-127 A rows, 128-255 W rows
  const int64_t sr = tid < kBM ? (m0 + tid < g.M ? m0 + tid : m0) : n0 + tid - kBM;
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wave < 2 ? g.sa : g.sw), 0, 0x7FFFFFFF, 0x00020000);
  const int svoff = (int)(sr * ngroups * SB);
  auto load_scale = [&](int s) -> uint32_t {
    const int gso = (s / SPG) * SB;
    return F16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs_s, svoff, gso, 0)
               : __builtin_amdgcn_raw_buffer_load_b32(rs_s, svoff, gso, 0);
  };

  // fragment read slots of K-step ks: piece 2 ks + h of row wm + l32 (+ 32 i)
  const int xr = (l32 / RPF) % SPR;
  int rd_a[STEPS], rd_b[STEPS];
#pragma unroll
  for (int ks = 0; ks < STEPS; ++ks) {
    rd_a[ks] = ((wm + l32) * SPR + ((2 * ks + h) ^ xr)) * 16;
    rd_b[ks] = OPB + ((wn + l32) * SPR + ((2 * ks + h) ^ xr)) * 16;
  }

  v16f c[2][2];
  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      c[i][j] = (v16f){};
      acc[i][j] = (v16i){};
    }

  auto mfma_half = [&](auto bufc, int i, bool zero_first, v4i (&bfr)[STEPS][2], bool read_b) {
    const char* sb = smem + decltype(bufc)::value * 2 * OPB;
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks) {
      const v4i af = *reinterpret_cast<const v4i*>(sb + rd_a[ks] + 32 * i * SPR * 16);
      if (read_b) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[ks][j] = *reinterpret_cast<const v4i*>(sb + rd_b[ks] + 32 * j * SPR * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = (zero_first && ks == 0)
                        ? __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bfr[ks][j], (v16i){}, 0, 0, 0)
                        : __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bfr[ks][j], acc[i][j], 0, 0, 0);
    }
  };
  // group epilogue of tiles (i, 0) and (i, 1), as in the packed kernel
  auto epilogue = [&](int i, int ring, int gi) {
    const char* ls = smem + LSC + ring * 1024;
    if (F16) {
      const uint32_t ra = *reinterpret_cast<const uint32_t*>(ls + (wm + 32 * i + l32) * 4) & hmask;
      const v4h sa = __builtin_bit_cast(v4h, (v2i){(int)ra, 0});
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t rw = *reinterpret_cast<const uint32_t*>(ls + (kBM + wn + 32 * j + l32) * 4) & hmask;
        const v4h sw = __builtin_bit_cast(v4h, (v2i){(int)rw, 0});
        const v16f p = __builtin_amdgcn_mfma_f32_32x32x8f16(sa, sw, (v16f){}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = fmaf((float)acc[i][j][v], p[v], c[i][j][v]);
      }
    } else {
      float sa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(ls + (wm + 32 * i + 8 * q + 4 * h) * 4);
        sa[4 * q] = __uint_as_float(t4.x);
        sa[4 * q + 1] = __uint_as_float(t4.y);
        sa[4 * q + 2] = __uint_as_float(t4.z);
        sa[4 * q + 3] = __uint_as_float(t4.w);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sw = *reinterpret_cast<const float*>(ls + (kBM + wn + 32 * j + l32) * 4);
#pragma unroll
        for (int v = 0; v < 16; ++v) c[i][j][v] = fmaf((float)acc[i][j][v], sa[v] * sw, c[i][j][v]);
      }
    }
    if (WRITE_ACC && gi >= 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const int64_t col = n0 + wn + 32 * j + l32;
          if (row < g.M) g.group_acc[(row * g.N + col) * ngroups + gi] = acc[i][j][v];
        }
    }
  };

  // one pipeline stage: the next stage's pieces and scale are requested
  // first and land during the two halves; the barrier at the end (with its
  // wait for them) makes them every wave's
  auto stage = [&](int s, auto bufc) {
    constexpr int B = decltype(bufc)::value;
    constexpr int SUB = SPG == 1 ? 0 : B;
    const int gi = s / SPG;
    const int ring = s % 3;
    // the last stage reloads itself (a valid address; the copy is never read)
    issue(s + 1 < nstages ? s + 1 : s, B ^ 1);
    const uint32_t psc = load_scale(s + 1 < nstages ? s + 1 : s);
    v4i bfr[STEPS][2];
    mfma_half(bufc, 0, SUB == 0, bfr, true);
    if (SUB == 0) epilogue(1, ring == 0 ? 2 : ring - 1, gi - 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 16, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_half(bufc, 1, SUB == 0, bfr, false);
    if (SUB == SPG - 1) epilogue(0, ring, gi);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    *reinterpret_cast<uint32_t*>(smem + LSC + (ring == 2 ? 0 : ring + 1) * 1024 + tid * 4) = psc;
    __syncthreads();
  };

  // ring slot 2 stands for the group before the first one: zero scales make
  // the lower tiles' first (empty) epilogue add nothing
  *reinterpret_cast<uint32_t*>(smem + LSC + 2 * 1024 + tid * 4) = 0u;
  issue(0, 0);
  *reinterpret_cast<uint32_t*>(smem + LSC + tid * 4) = load_scale(0);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= nstages; s += 2) {
    stage(s, IntC<0>{});
    stage(s + 1, IntC<1>{});
  }
  if (s < nstages) stage(s, IntC<0>{});
  epilogue(1, (nstages - 1) % 3, ngroups - 1);

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < g.M) {
#pragma unroll
        for (int j = 0; j < 2; ++j) g.c[row * g.N + n0 + wn + 32 * j + l32] = c[i][j][v];
      }
    }
}

// M <= 16: each workgroup owns 16 output columns; its 16 waves split K.  The
// unit of work is a 64-byte run of a packed row (128 codes), or two runs when
// a group spans two (G = 256); wave w takes units [w U / 16, (w + 1) U / 16).
// Time here is set by how many bytes each CU pulls in (every workgroup also
// reads the 16 rows of A), so a wave issues all loads of a chunk of CH runs
// at once, with global_load_lds so that no registers wait on them: lane l of
// a load reads row l / 4, 16-byte piece (l % 4) ^ ((l / 16) % 4) of the run,
// four lanes covering 64 contiguous bytes.  A run feeds two
// v_mfma_i32_16x16x64_i8 (codes 0..63 and 64..127); lane (r, j) = (lane % 16,
// lane / 16) reads the 8 bytes of codes 16 j .. 16 j + 15 of that half (same K
// slots for A and W, so group sums stay exact) with one ds_read_b64, and the
// piece XOR spreads the 16 rows over all LDS banks.  The 16 partial 16 x 16
// tiles are summed through LDS.
//
// W4A8: an A run is 128 bytes; two loads cover its 16 rows (lane l of load i
// reads row 8 i + l / 8, piece (l % 8) ^ ((row / 2) % 8): eight lanes per 128
// contiguous bytes), and lane (r, j) reads its 16 codes of half h as one
// ds_read_b128 of piece 4 h + j, reordered with v_perm_b32.
//
// G = 32: a group is one 16-byte piece of a packed run (32 codes) and one
// v_mfma_i32_16x16x32_i8; lane (r, j) takes dword j of the piece (8 codes,
// unpacked to the same even/odd K order on both operands), or for int8
// activations the 8 bytes 8 j .. 8 j + 7 of the group.
constexpr int kDecWaves = 16;
constexpr int kDecRuns = 2;      // runs per operand and chunk

__device__ __forceinline__ void dec_lds_load16(const void* gp, void* lp) {
  __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
}
__device__ __forceinline__ void dec_wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int G, bool F16, bool WRITE_ACC, bool A8>
__global__ __launch_bounds__(kDecWaves * 64) void w4a4_gemm_decode_kernel(GemmArgs g) {
  constexpr int CH = kDecRuns;
  constexpr int MPG = G >= 64 ? G / 64 : 1;      // MFMAs per group (G = 32: one 16x16x32)
  constexpr int RPU = G >= 128 ? G / 128 : 1;    // runs per unit of work
  constexpr int GPC = G >= 64 ? 2 * CH / MPG : 4 * CH;   // groups per chunk
  typedef typename std::conditional<F16, _Float16, float>::type scale_t;
  __shared__ float part[kDecWaves][16 * 16];
  __shared__ __attribute__((aligned(16))) float sat[kDecWaves][GPC][16];   // [group][A row]
  __shared__ __attribute__((aligned(16))) uint4 stage_w[kDecWaves][CH][64];
  __shared__ __attribute__((aligned(16))) uint4 stage_a4[A8 ? 1 : kDecWaves][CH][64];
  __shared__ __attribute__((aligned(16))) uint4 stage_a8[A8 ? kDecWaves : 1][CH][128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t rowb = g.K / 2;
  const int64_t rowb_a = A8 ? g.K : rowb;
  const int ngroups = (int)(g.K / G);
  const int units = (int)(g.K / (128 * RPU));
  const int rbeg = RPU * (wave * units / kDecWaves), rend = RPU * ((wave + 1) * units / kDecWaves);
  const bool arow = r < g.M;
  // loads: row l / 4, piece (l % 4) ^ ((l / 16) % 4)
  const int lrow = lane >> 2, lpiece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint8_t* la = g.a + (int64_t)(lrow < g.M ? lrow : 0) * rowb + 16 * lpiece;
  // int8 A: load i reads row 8 i + l / 8, piece (l % 8) ^ ((row / 2) % 8)
  const int arow0 = lane >> 3, arow1 = 8 + (lane >> 3);
  const uint8_t* la8_0 = g.a + (int64_t)(arow0 < g.M ? arow0 : 0) * rowb_a +
                         16 * ((lane & 7) ^ ((arow0 >> 1) & 7));
  const uint8_t* la8_1 = g.a + (int64_t)(arow1 < g.M ? arow1 : 0) * rowb_a +
                         16 * ((lane & 7) ^ ((arow1 >> 1) & 7));
  const uint32_t rd8 = 16u * (uint32_t)(8 * r);   // + 16 * ((4 h + j) ^ ((r / 2) % 8))
  const uint8_t* lw = g.w + (n0 + lrow) * rowb + 16 * lpiece;
  // reads, half h of a run: piece 2 h + j / 2, byte 8 (j % 2) of it
  const uint32_t rd0 = 64 * r + 16 * ((0 + (j >> 1)) ^ ((r >> 2) & 3)) + 8 * (j & 1);
  const uint32_t rd1 = 64 * r + 16 * ((2 + (j >> 1)) ^ ((r >> 2) & 3)) + 8 * (j & 1);
  const int64_t sa_row = (int64_t)(arow ? r : 0) * ngroups, sw_row = (n0 + r) * ngroups;
  float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r0 = rbeg; r0 < rend; r0 += CH) {
    const int nr = rend - r0 < CH ? rend - r0 : CH;    // runs in this chunk (>= 1)
    const int g0 = r0 * 128 / G;                       // first group of the chunk
    const int ng = (nr * 128 + G - 1) / G;             // groups in this chunk
    // every load is issued (indices past the chunk repeat its last run or
    // group, in bounds) so that none waits behind a branch
    scale_t sab[GPC], swb[GPC];
#pragma unroll
    for (int u = 0; u < GPC; ++u) {
      const int uu = u < ng ? u : ng - 1;
      sab[u] = reinterpret_cast<const scale_t*>(g.sa)[sa_row + g0 + uu];
      swb[u] = reinterpret_cast<const scale_t*>(g.sw)[sw_row + g0 + uu];
    }
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int64_t run = r0 + (t < nr ? t : nr - 1);
      if (A8) {
        dec_lds_load16(la8_0 + run * 128, &stage_a8[wave][t][0]);
        dec_lds_load16(la8_1 + run * 128, &stage_a8[wave][t][64]);
      } else {
        dec_lds_load16(la + run * 64, &stage_a4[wave][t][0]);
      }
      dec_lds_load16(lw + run * 64, &stage_w[wave][t][0]);
    }
    dec_wait_loads();
    // A scales transposed through this wave's LDS: lane reads rows 4 j .. 4 j + 3
    if (j == 0) {
#pragma unroll
      for (int u = 0; u < GPC; ++u)
        if (u < ng) sat[wave][u][r] = arow ? (float)sab[u] : 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
    const char* sta = reinterpret_cast<const char*>(&stage_a4[A8 ? 0 : wave][0][0]);
    const char* stw = reinterpret_cast<const char*>(&stage_w[wave][0][0]);
#pragma unroll
    for (int u = 0; u < GPC; ++u) {
      if (u >= ng) break;
      v4i acc = (v4i){0, 0, 0, 0};
      if (G == 32) {
        // group u: piece p = u % 4 of run u / 4; W (and packed A) dword j of
        // row r's piece, int8 A bytes 8 j .. 8 j + 7 of the group
        const int run = u >> 2, p = u & 3;
        const uint32_t o = 1024u * run + 64u * r + 16u * (p ^ ((r >> 2) & 3)) + 4u * j;
        const uint32_t pw = *reinterpret_cast<const uint32_t*>(stw + o);
        uint2 av;
        if (A8) {
          const int pc = (2 * p + (j >> 1)) ^ ((r >> 1) & 7);
          const uint2 pa = *reinterpret_cast<const uint2*>(
              reinterpret_cast<const char*>(&stage_a8[wave][run][0]) + rd8 + 16 * pc + 8 * (j & 1));
          av = arow ? make_uint2(__builtin_amdgcn_perm(pa.y, pa.x, 0x06040200u),
                                 __builtin_amdgcn_perm(pa.y, pa.x, 0x07050301u))
                    : make_uint2(0u, 0u);
        } else {
          const uint32_t pa = arow ? *reinterpret_cast<const uint32_t*>(sta + o) : 0u;
          av = make_uint2((pa << 4) & 0xF0F0F0F0u, pa & 0xF0F0F0F0u);
        }
        const uint2 wv = make_uint2((pw << 4) & 0xF0F0F0F0u, pw & 0xF0F0F0F0u);
        acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, av),
                                                    __builtin_bit_cast(long, wv), acc, 0, 0, 0);
      }
#pragma unroll
      for (int m = u * MPG; G >= 64 && m < (u + 1) * MPG; ++m) {
        const uint32_t o = 1024u * (m >> 1) + ((m & 1) ? rd1 : rd0);
        const uint2 pw = *reinterpret_cast<const uint2*>(stw + o);
        v4i av;
        if (A8) {
          const int pc = (4 * (m & 1) + j) ^ ((r >> 1) & 7);
          const uint4 pa = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const char*>(&stage_a8[wave][m >> 1][0]) + rd8 + 16 * pc);
          av = arow ? order_int8(pa) : (v4i){0, 0, 0, 0};
        } else {
          const uint2 pa = *reinterpret_cast<const uint2*>(sta + o);
          av = unpack16(make_uint2(arow ? pa.x : 0u, arow ? pa.y : 0u));
        }
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, unpack16(pw), acc, 0, 0, 0);
      }
      // lane holds rows 4 j + v of column n0 + r
      const float sw = (float)swb[u] * (A8 ? 1.0f / 16.0f : 1.0f / 256.0f);
      const float4 s4 = *reinterpret_cast<const float4*>(&sat[wave][u][4 * j]);
      const float sar[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        c[v] = fmaf((float)acc[v], sar[v] * sw, c[v]);
        if (WRITE_ACC) {
          const int row = 4 * j + v;
          if (row < g.M)
            g.group_acc[((int64_t)row * g.N + n0 + r) * ngroups + g0 + u] = acc[v] >> (A8 ? 4 : 8);
        }
      }
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
      for (int w = 0; w < kDecWaves; ++w) s += part[w][tid];
      g.c[(int64_t)row * g.N + n0 + col] = s;
    }
  }
}

template <int G, bool F16, bool WRITE_ACC, bool A8>
static void launch_g(const GemmArgs& a, hipStream_t s) {
  // G = 32 reaches this only with M <= 16 (launch_gemm_mfma)
  if (a.M <= 16) {
    hipLaunchKernelGGL((w4a4_gemm_decode_kernel<G, F16, WRITE_ACC, A8>), dim3((unsigned)(a.N / 16)),
                       dim3(kDecWaves * 64), 0, s, a);
  } else if constexpr (G >= 64) {
    const dim3 grid((unsigned)(a.N / kBN), (unsigned)((a.M + kBM - 1) / kBM));
    hipLaunchKernelGGL((w4a4_gemm_tile_kernel<G, F16, WRITE_ACC, A8>), grid, dim3(256), 0, s, a);
  }
}

template <int G, bool A8>
static void launch_dt(const GemmArgs& a, hipStream_t s) {
  if (a.scale_f16) {
    if (a.group_acc) launch_g<G, true, true, A8>(a, s); else launch_g<G, true, false, A8>(a, s);
  } else {
    if (a.group_acc) launch_g<G, false, true, A8>(a, s); else launch_g<G, false, false, A8>(a, s);
  }
}

template <int G>
static void launch_da(const GemmArgs& a, hipStream_t s) {
  if (a.a_int8) launch_dt<G, true>(a, s); else launch_dt<G, false>(a, s);
}

// The prefill kernel needs N % 128 == 0; the decode kernel takes every shape
// the library accepts (N % 64 == 0, K a multiple of 256 and of the group).
// Other shapes go to the simple kernel.
template <int G, bool F16>
static void launch_w8(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.N / kBN), (unsigned)((a.M + kBM - 1) / kBM));
  if (a.group_acc)
    hipLaunchKernelGGL((w8a8_gemm_tile_kernel<G, F16, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((w8a8_gemm_tile_kernel<G, F16, false>), grid, dim3(256), 0, s, a);
}

template <int G>
static void launch_w8g(const GemmArgs& a, hipStream_t s) {
  if (a.scale_f16) launch_w8<G, true>(a, s); else launch_w8<G, false>(a, s);
}

bool launch_gemm_mfma(const GemmArgs& a, hipStream_t s) {
  if (a.w_int8) {
    // int8 weights: the tile kernel for M > 16 and N % 128 == 0, else the
    // simple kernel
    if (!a.a_int8 || a.M <= 16 || a.N % kBN) return false;
    switch (a.group) {
      case 64: launch_w8g<64>(a, s); return true;
      case 128: launch_w8g<128>(a, s); return true;
      case 256: launch_w8g<256>(a, s); return true;
      default: return false;
    }
  }
  const bool decode = a.M <= 16;
  if (!decode && a.N % kBN) return false;
  switch (a.group) {
    case 32:
      // G = 32 has a kernel for M <= 16 only; the simple kernel takes M > 16
      if (!decode) return false;
      launch_da<32>(a, s);
      return true;
    case 64: launch_da<64>(a, s); return true;
    case 128: launch_da<128>(a, s); return true;
    case 256: launch_da<256>(a, s); return true;
    default: return false;
  }
}

}  // namespace hr
