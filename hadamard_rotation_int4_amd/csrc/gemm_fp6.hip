// W4A4 GEMM on fp6 matrix cores, and the conversion of packed int4 codes to
// the operand format it reads.
//
// What is computed ("Experiment -- Hadamard rotation for int4 (W4A4)
// accuracy", Hypothesis and Verdict): C = A W^T with
//   acc[m][n][g] = sum_{k in group g} a[m][k] w[n][k]   (exact)
//   C[m][n]      = sum_g sA[m][g] sW[n][g] acc[m][n][g]  (fp32)
// as hr_w4a4_gemm, on operands held in the fp6 slot format below.
//
// Why fp6.  A code q in [-8, 7] written sign-magnitude into the 6-bit e2m3
// format (sign bit 5, the 5 low bits |q|) is the value q / 8: magnitudes 0..7
// are the format's subnormals (|q| x 2^-3) and 8 is its smallest normal
// (1.0).  Every product of two such values is a multiple of 2^-6 below 1, and
// the fp32 accumulation of a group's products (at most 256 x 64 / 64) is exact,
// so v_mfma_f32_32x32x64_f8f6f4 returns each group sum as S / 64 in fp32
// without rounding -- the int32 sum of the int8 kernels, already converted.
// The epilogue is then one fma per output and group (the int8 kernels need a
// conversion as well), and the fp6 matrix rate is twice the int8 rate on
// gfx950.
//
// Tiled fp6 format.  A slot is 32 consecutive codes of a row, 24 bytes, code
// 32 j + e (e < 32) of the slot in bits 6 e .. 6 e + 5 of its 192-bit
// little-endian value.  Rows go in panels of 128 (the last one padded with
// zero rows), K in blocks of 128 codes (four slots); panel p, block b is a
// 12288-byte tile at ((p * K / 128) + b) * 12288, made of two planes of 6144
// bytes: plane h holds, for each row r of the panel, slots h and h + 2 of the
// block at h * 6144 + r * 48.  The tile is exactly the LDS image the GEMM
// reads (a lane of an MFMA K-step pair needs slots h and h + 2), so the GEMM
// loads it with plain 1 KB copies, eight whole cache lines each.  The scales
// that go with a tiled operand are transposed, [K / G][padded rows], zeros for
// the padding rows.
#include "hr_internal.h"
#include "hr_device.h"

namespace hr {

typedef int f6_v8i __attribute__((ext_vector_type(8)));
typedef float f6_v16f __attribute__((ext_vector_type(16)));
typedef _Float16 f6_v4h __attribute__((ext_vector_type(4)));
typedef int f6_v2i __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- conversion

// (f6_fields8, which turns 8 packed int4 codes into 8 fp6 fields, is in
// hr_device.h: the fp6-output rotation kernel uses it too)

// One workgroup of 256 threads per output tile (panel p = blockIdx.y, block
// kb = blockIdx.x): thread t writes row r = t % 128 of plane h = t / 128, the
// 48 contiguous bytes of slots h and h + 2 of that row's block (zeros for the
// padding rows of the last panel), so a wave writes 3 KB of the tile in one
// run.  The tile holding a group's first codes also writes the panel's 128
// transposed scales of that group.
template <typename S>
__global__ __launch_bounds__(256) void int4_to_fp6_kernel(const uint8_t* __restrict__ codes, int64_t rows,
                                                         int64_t K, uint8_t* __restrict__ out,
                                                         const S* __restrict__ scales, int group,
                                                         S* __restrict__ out_scales) {
  const int t = threadIdx.x;
  const int r = t & 127, h = t >> 7;
  const int64_t p = blockIdx.y, kb = blockIdx.x;
  const int64_t row = p * 128 + r;
  const int64_t nkb = K / 128;
  uint4 x0 = make_uint4(0u, 0u, 0u, 0u), x1 = x0;
  if (row < rows) {
    // slots h and h + 2 of the block: packed bytes 16 h and 16 (h + 2) of its 64
    const uint4* src = reinterpret_cast<const uint4*>(codes + row * (K / 2) + kb * 64);
    x0 = src[h];
    x1 = src[h + 2];
  }
  auto fields = [](const uint4& x, uint32_t (&o)[6]) {
    const uint64_t f0 = f6_fields8(x.x), f1 = f6_fields8(x.y), f2 = f6_fields8(x.z), f3 = f6_fields8(x.w);
    // 192 bits: f0 | f1 << 48 | f2 << 96 | f3 << 144
    o[0] = (uint32_t)f0;
    o[1] = (uint32_t)(f0 >> 32) | ((uint32_t)f1 << 16);
    o[2] = (uint32_t)(f1 >> 16);
    o[3] = (uint32_t)f2;
    o[4] = (uint32_t)(f2 >> 32) | ((uint32_t)f3 << 16);
    o[5] = (uint32_t)(f3 >> 16);
  };
  uint32_t a[6], b[6];
  fields(x0, a);
  fields(x1, b);
  uint4* dst = reinterpret_cast<uint4*>(out + (p * nkb + kb) * 12288 + h * 6144 + r * 48);
  dst[0] = make_uint4(a[0], a[1], a[2], a[3]);
  dst[1] = make_uint4(a[4], a[5], b[0], b[1]);
  dst[2] = make_uint4(b[2], b[3], b[4], b[5]);
  // the tile that holds a group's first codes writes that group's 128
  // transposed scales of the panel: out_scales[g][p * 128 + r]
  if (scales && t < 128 && (kb * 128) % group == 0) {
    const int64_t g = kb * 128 / group, ngroups = K / group;
    const int64_t prow = (int64_t)gridDim.y * 128;
    out_scales[g * prow + row] = row < rows ? scales[row * ngroups + g] : S(0);
  }
}

hipError_t launch_int4_to_fp6(const uint8_t* codes, const void* scales, bool scale_f16, int64_t rows, int64_t K,
                              int group, uint8_t* out, void* out_scales, hipStream_t s) {
  const dim3 grid((unsigned)(K / 128), (unsigned)((rows + 127) / 128));
  const int g = scales ? group : 128;   // unused without scales
  if (!scales || scale_f16)
    hipLaunchKernelGGL(int4_to_fp6_kernel<uint16_t>, grid, dim3(256), 0, s, codes, rows, K, out,
                       static_cast<const uint16_t*>(scales), g, static_cast<uint16_t*>(out_scales));
  else
    hipLaunchKernelGGL(int4_to_fp6_kernel<uint32_t>, grid, dim3(256), 0, s, codes, rows, K, out,
                       static_cast<const uint32_t*>(scales), g, static_cast<uint32_t*>(out_scales));
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM

template <int V>
struct F6C { static constexpr int value = V; };

// Workgroup barrier that leaves loads in flight.  The compiler puts a wait for
// every outstanding memory operation in front of each s_barrier it emits,
// which would drain the loads of the stage after next; written as inline asm
// the barrier keeps the caller's own (partial) wait.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void f6_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kF6BM = 128, kF6BN = 128;
constexpr int kF6SchedValu = 0x2, kF6SchedMfma = 0x8, kF6SchedDsRead = 0x100;

// A 128 x 128 output tile per workgroup of 4 waves, 64 x 64 per wave as 2 x 2
// tiles of v_mfma_f32_32x32x64_f8f6f4 (fp6 e2m3 operands).
//
// Pipeline.  A stage is one 128-code block: one tile per operand, copied from
// memory straight into LDS with buffer loads to LDS (1 KB per instruction).  Three stage buffers, each its own LDS
// array: stage s reads buffer s % 3 while the loads of stage s + 2 fill buffer
// (s + 2) % 3, and at its end waits only for the loads of stage s + 1.  What
// keeps the compiler from draining the loads early: the buffers are separate
// arrays (so it can see that a read of one does not depend on loads into
// another); nothing is stored to LDS inside the loop (it orders every LDS
// store after all LDS loads in flight); the loads are buffer loads, not
// global_load_lds (a pending instruction of the flat family that touches LDS
// makes it wait for everything); and the barrier is its own.
//
// LDS image.  A stage's image of an operand is its 12288-byte tile of the
// tiled format: lane (row l % 32, half h = l / 32) needs slots h and h + 2 of
// its row (the fragments of both K-steps), which plane h holds at row * 48, so
// a lane reads its fragments with three ds_read_b128 from one address.  The 16
// lanes of one pass of a read (consecutive rows, one plane) hit 16-byte bank
// groups 3 r + t mod 16, all distinct.
//
// Scales.  The scales come transposed ([group][row], from the converter), so
// the 128 scales of a panel and group are 256 (f16) or 512 (f32) contiguous
// bytes: each wave copies 256 of them per stage, with the tiles, into the end
// of the stage's buffer.  The epilogue of the lower tiles runs a stage late;
// the three scales it needs are carried over in registers, so that a buffer
// is free once its stage ends.
//
// Epilogue.  The outer product sA x sW of a 32 x 32 tile comes from one MFMA
// with K = 8 (f16) or 2 (f32) whose only non-zero K index is 0 (lanes 32-63
// pass zeros), then one fma per output; the MFMAs of one pair of tiles
// overlap the epilogue of the other pair.
template <int G, bool F16, bool WRITE_ACC>
__global__ __launch_bounds__(256, 2) void w4a4_gemm_fp6_tile_kernel(GemmArgs g) {
  static_assert(G == 128 || G == 256, "stages of 128 codes, one group per stage or two stages per group");
  constexpr int KS = 128;                 // codes per row and stage
  constexpr int STEPS = KS / 64;          // MFMA K-steps per stage
  constexpr int SPG = G / KS;             // stages per group (1 or 2)
  constexpr int RB = KS * 3 / 4;          // bytes per row and stage (96)
  constexpr int OPB = 128 * RB;           // bytes of one operand stage (a tile)
  static_assert(OPB == 12288, "tile size of the tiled format");
  constexpr int NQ = OPB / 1024;          // load instructions per operand and stage
  constexpr int DPW = 2 * NQ / 4;         // ... per wave (both operands)
  constexpr int SB = F16 ? 2 : 4;
  static_assert(DPW + 1 < 16, "vmcnt immediate");
  constexpr int LSC = 2 * OPB;            // offset of the scales in a stage buffer
  __shared__ __attribute__((aligned(16))) char sbuf0[LSC + 256 * SB];   // A tile, W tile, [operand][row] scales
  __shared__ __attribute__((aligned(16))) char sbuf1[LSC + 256 * SB];
  __shared__ __attribute__((aligned(16))) char sbuf2[LSC + 256 * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.y * kF6BM;
  const int64_t n0 = (int64_t)blockIdx.x * kF6BN;
  const int64_t K = g.K;
  const int ngroups = (int)(K / G);
  const int nstages = (int)(K / KS);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // this workgroup's panels of A and W (A's padding rows are zeros)
  const int64_t tile_stride = (int64_t)nstages * OPB;
  const uint8_t* pa = g.a + (int64_t)blockIdx.y * tile_stride;
  const uint8_t* pw = g.w + (int64_t)blockIdx.x * tile_stride;
  auto buf = [&](auto bc) -> char* {
    if constexpr (decltype(bc)::value == 0) return sbuf0;
    else if constexpr (decltype(bc)::value == 1) return sbuf1;
    else return sbuf2;
  };
  // stage s's tiles into buffer bc: load instruction j of this wave copies KB
  // q % NQ of operand q / NQ (q = DPW wave + j).  keep = 0 turns the loads
  // into copies of the tile's first 16 bytes (one cache line), which nothing
  // reads: every stage then issues the same number of loads, which the
  // stage-end wait counts on.
  const __amdgpu_buffer_rsrc_t rs_pa = __builtin_amdgcn_make_buffer_rsrc((void*)pa, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_pw = __builtin_amdgcn_make_buffer_rsrc((void*)pw, 0, 0x7FFFFFFF, 0x00020000);
  auto issue = [&](int s, auto bc, int keep) {
    char* b = buf(bc);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int q = DPW * wave + j;
      const int op = q / NQ;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(op == 0 ? rs_pa : rs_pw,
          (__attribute__((address_space(3))) void*)(b + op * OPB + 1024 * (q % NQ)), 16,
          (1024 * (q % NQ) + 16 * lane) & keep, s * OPB, 0, 0);
    }
  };

  // this wave's 256 bytes of a stage's scales: chunk (F16: wave % 2, F32:
  // wave) of operand chunk / (SB / 2), part chunk % (SB / 2)
  const int chunk = F16 ? (wave & 1) : wave;
  const int sop = chunk / (SB / 2), spart = chunk % (SB / 2);
  const int64_t prow = sop == 0 ? (int64_t)gridDim.y * kF6BM : g.N;   // rows of the transposed array
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)(sop == 0 ? g.sa : g.sw) + ((sop == 0 ? m0 : n0) * SB + spart * 256)), 0, 0x7FFFFFFF,
      0x00020000);
  auto issue_scales = [&](int s, auto bc) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs_s, (__attribute__((address_space(3))) void*)(buf(bc) + LSC + sop * 128 * SB + spart * 256), 4,
        4 * lane, (int)((s / SPG) * prow * SB), 0, 0);
  };

  f6_v16f c[2][2], acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      c[i][j] = (f6_v16f){};
      acc[i][j] = (f6_v16f){};
    }

  // both K-steps' fragments of lane (row, h): plane h, row row
  auto frag2 = [&](const char* sb, int row, f6_v8i (&f)[2]) {
    const uint4* rp = reinterpret_cast<const uint4*>(sb + h * (OPB / 2) + row * (RB / 2));
    const uint4 x0 = rp[0], x1 = rp[1], x2 = rp[2];
    f[0] = (f6_v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, 0, 0};
    f[1] = (f6_v8i){(int)x1.z, (int)x1.w, (int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w, 0, 0};
  };
  auto mfma_tiles = [&](int i, bool zero_first, const f6_v8i (&af)[STEPS], const f6_v8i (&bfr)[2][STEPS]) {
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            af[ks], bfr[j][ks], (zero_first && ks == 0) ? (f6_v16f){} : acc[i][j], 2, 2, 0, 0, 0, 0);
  };
  // a stage's scales for this lane, as raw bits: sA of rows wm + l32 and
  // wm + 32 + l32, sW of columns wn + l32 and wn + 32 + l32
  struct Scales { uint32_t a[2], w[2]; };
  auto read_scales = [&](auto bc) -> Scales {
    const char* ls = buf(bc) + LSC;
    Scales r;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (F16) {
        r.a[t] = *reinterpret_cast<const uint16_t*>(ls + (wm + 32 * t + l32) * 2);
        r.w[t] = *reinterpret_cast<const uint16_t*>(ls + 256 + (wn + 32 * t + l32) * 2);
      } else {
        r.a[t] = *reinterpret_cast<const uint32_t*>(ls + (wm + 32 * t + l32) * 4);
        r.w[t] = *reinterpret_cast<const uint32_t*>(ls + 512 + (wn + 32 * t + l32) * 4);
      }
    }
    return r;
  };
  // group epilogue of tiles (i, 0) and (i, 1) with sA bits ra and sW bits rw;
  // lane holds acc[i][j][v] of row wm + 32 i + 8 (v / 4) + 4 h + v % 4, column
  // wn + 32 j + l32, and p[v] of the outer product is the same entry's sA sW
  auto epilogue = [&](int i, uint32_t ra, const uint32_t (&rw)[2], int gi) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f6_v16f p;
      if constexpr (F16) {
        const f6_v4h sa = __builtin_bit_cast(f6_v4h, (f6_v2i){(int)(h ? 0u : ra), 0});
        const f6_v4h sw = __builtin_bit_cast(f6_v4h, (f6_v2i){(int)(h ? 0u : rw[j]), 0});
        p = __builtin_amdgcn_mfma_f32_32x32x8f16(sa, sw, (f6_v16f){}, 0, 0, 0);
      } else {
        p = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 0.0f : __uint_as_float(ra), h ? 0.0f : __uint_as_float(rw[j]),
                                                 (f6_v16f){}, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) c[i][j][v] = fmaf(acc[i][j][v], p[v], c[i][j][v]);
    }
    if (WRITE_ACC && gi >= 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const int64_t col = n0 + wn + 32 * j + l32;
          // acc holds S / 64 exactly
          if (row < g.M) g.group_acc[(row * g.N + col) * ngroups + gi] = (int32_t)(acc[i][j][v] * 64.0f);
        }
    }
  };

  // scales of the previous stage for the delayed epilogue (zeros before the
  // first stage: its lower tiles' epilogue adds nothing)
  uint32_t prev_a = 0u, prev_w[2] = {0u, 0u};

  // stage s, read from buffer B = s % 3; SUB = s % SPG
  auto stage = [&](int s, auto bc, auto subc) {
    constexpr int B = decltype(bc)::value;
    constexpr int SUB = decltype(subc)::value;
    const int gi = s / SPG;
    const char* sb = buf(bc);
    f6_v8i af[STEPS], bfr[2][STEPS];
    frag2(sb, wm + l32, af);
#pragma unroll
    for (int j = 0; j < 2; ++j) frag2(sb + OPB, wn + 32 * j + l32, bfr[j]);
    // stage s + 2's tiles and scales (past the last stage, the dummy loads of
    // issue() into a buffer nothing reads, and stage s's scales again into a
    // ring slot nothing reads)
    const bool more = s + 2 < nstages;      // uniform
    issue(more ? s + 2 : 0, F6C<(B + 2) % 3>{}, more ? -1 : 0);
    issue_scales(more ? s + 2 : s, F6C<(B + 2) % 3>{});
    mfma_tiles(0, SUB == 0, af, bfr);
    if (SUB == 0) epilogue(1, prev_a, prev_w, gi - 1);
    __builtin_amdgcn_sched_group_barrier(kF6SchedDsRead, 9, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kF6SchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kF6SchedValu, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    frag2(sb, wm + 32 + l32, af);
    const Scales sc = read_scales(bc);
    mfma_tiles(1, SUB == 0, af, bfr);
    if (SUB == SPG - 1) epilogue(0, sc.a[0], sc.w, gi);
    prev_a = sc.a[1];
    prev_w[0] = sc.w[0];
    prev_w[1] = sc.w[1];
    __builtin_amdgcn_sched_group_barrier(kF6SchedDsRead, 7, 0);
#pragma unroll
    for (int q = 0; q < 2 * STEPS + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(kF6SchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kF6SchedValu, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the loads of stage s + 1 (issued one stage earlier) have landed; this
    // stage's DPW + 1 may still be in flight.  Loads complete in order, so at
    // most DPW + 1 outstanding means all older ones are done.
    __builtin_amdgcn_s_waitcnt(0x0070 | (DPW + 1));   // vmcnt(DPW + 1) lgkmcnt(0)
    f6_barrier();
  };

  issue(0, F6C<0>{}, -1);
  issue_scales(0, F6C<0>{});
  issue(nstages > 1 ? 1 : 0, F6C<1>{}, nstages > 1 ? -1 : 0);
  issue_scales(nstages > 1 ? 1 : 0, F6C<1>{});
  __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  // unrolled by 3 SPG stages, so that both the buffer and the position in the
  // group are compile-time constants; nstages is a multiple of SPG
  int s = 0;
  for (; s + 3 * SPG <= nstages; s += 3 * SPG) {
    stage(s, F6C<0>{}, F6C<0>{});
    stage(s + 1, F6C<1>{}, F6C<1 % SPG>{});
    stage(s + 2, F6C<2>{}, F6C<2 % SPG>{});
    if constexpr (SPG == 2) {
      stage(s + 3, F6C<0>{}, F6C<1>{});
      stage(s + 4, F6C<1>{}, F6C<0>{});
      stage(s + 5, F6C<2>{}, F6C<1>{});
    }
  }
  if (s < nstages) stage(s, F6C<0>{}, F6C<0>{});
  if (s + 1 < nstages) stage(s + 1, F6C<1>{}, F6C<1 % SPG>{});
  if constexpr (SPG == 2) {
    if (s + 2 < nstages) stage(s + 2, F6C<2>{}, F6C<0>{});
    if (s + 3 < nstages) stage(s + 3, F6C<0>{}, F6C<1>{});
  }
  // the last stage's (dummy) loads must land before the workgroup's LDS is
  // given to another one
  __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0)
  epilogue(1, prev_a, prev_w, ngroups - 1);

  // each product of two fp6 codes is (q_a / 8)(q_w / 8): the sums are 1/64 of
  // the true ones
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < g.M) {
#pragma unroll
        for (int j = 0; j < 2; ++j) g.c[row * g.N + n0 + wn + 32 * j + l32] = c[i][j][v] * 64.0f;
      }
    }
}

template <int G, bool F16>
static void launch_f6(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.N / kF6BN), (unsigned)((a.M + kF6BM - 1) / kF6BM));
  if (a.group_acc)
    hipLaunchKernelGGL((w4a4_gemm_fp6_tile_kernel<G, F16, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((w4a4_gemm_fp6_tile_kernel<G, F16, false>), grid, dim3(256), 0, s, a);
}

template <int G>
static void launch_f6g(const GemmArgs& a, hipStream_t s) {
  if (a.scale_f16) launch_f6<G, true>(a, s); else launch_f6<G, false>(a, s);
}

hipError_t launch_gemm_fp6(const GemmArgs& a, hipStream_t s) {
  if (a.group == 128) launch_f6g<128>(a, s);
  else launch_f6g<256>(a, s);
  return hipGetLastError();
}

}  // namespace hr
