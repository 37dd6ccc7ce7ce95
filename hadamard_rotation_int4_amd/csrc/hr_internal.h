// Internal declarations shared by the HIP translation units of libhr.so.
// Nothing here is part of the public ABI (include/hr.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hr {

// Inputs at least this large are read with the nontemporal hint.  Streamed
// once from HBM they are faster with it (bf16 65536 x 2048 rotation: 62.9
// against 63.8 us; the rotation-free quantizer 57.4 against 63.8 us); a
// smaller input may still sit in the 256 MB last-level cache from whatever
// wrote it, and the hint then costs (bf16 4096 x 4096 rotation read again
// each call: 14.3 against 12.9 us).  A quarter of that cache, same box.
constexpr int64_t kStreamBytes = int64_t(64) << 20;

// Arguments of one rotate / rotate+quantize call after host validation.
struct RhtArgs {
  const void* x;
  int x_bf16;            // 1: bf16 input, 0: fp32 input
  int64_t rows;
  int n, m, p;           // n = m * p
  const int8_t* signs;   // may be null (all +1)
  const float* block;    // [m][m], null when m == 1
  float* y;              // fp32 output or null
  int group;             // quantization group (when codes != null)
  uint8_t* codes;        // packed int4 (bits 4), int8 (bits 8) or tiled fp6 (bits 6) codes, or null
  int bits;              // 4, 8 or 6 (when codes != null)
  void* scales;          // scale output or null
  int scale_f16;         // 1: fp16 scales, 0: fp32 scales
};

// Arguments of one rotation-free quantize call after host validation.
struct QuantArgs {
  const void* x;
  int x_bf16;            // 1: bf16 input, 0: fp32 input
  int64_t rows;
  int n;                 // a multiple of group
  int group;
  int bits;              // 4 (packed int4 codes) or 8 (int8 codes)
  uint8_t* codes;
  void* scales;
  int scale_f16;
};

struct ButterflyArgs {
  const float* x;
  float* y;
  int64_t rows;
  int n, log2n;
  const float* coeffs;   // [log2 n][n/2][2]
  int precondition;
  const int* perm;
  int inverse;
  int group;
  uint8_t* codes;
  void* scales;
  int scale_f16;
};

struct GemmArgs {
  const uint8_t* a;      // packed int4 [M][K/2], or int8 [M][K] when a_int8
  int a_int8;            // 1: int8 activation codes [M][K] (W4A8, W8A8)
  int w_int8;            // 1: int8 weight codes [N][K] (W8A8)
  const void* sa;
  const uint8_t* w;
  const void* sw;
  int scale_f16;
  int64_t M, N, K;
  int group;
  float* c;
  int32_t* group_acc;
};

// Arguments of the fused decode call (rotation + int4 quantization of M <= 16
// bf16 rows, then the W4A4 GEMM on the codes) after host validation.
struct FusedDecodeArgs {
  const uint16_t* x;     // bf16 [M][K]
  const int8_t* signs;   // [K] or null
  float norm;            // 1 / sqrt(K)
  const uint8_t* w;      // packed int4 [N][K/2]
  const void* sw;        // [N][K/G]
  int scale_f16;
  int64_t M, N, K;
  int group;
  float* c;              // [M][N]
  uint8_t* a_codes;      // optional [M][K/2] copy of the activation codes
  void* a_scales;        // optional [M][K/G] copy of their scales
};

constexpr int kHarpMaxStages = 16;
constexpr int kHarpMaxRadix = 8;

// A mixed-radix schedule with its per-stage offsets (filled on the host).
struct HarpSchedule {
  int nstages;
  int radix[kHarpMaxStages];
  int stride[kHarpMaxStages];               // b_0 ... b_{t-1}
  int64_t block_begin[kHarpMaxStages + 1];  // global index of the first block of each stage
  int64_t theta_off[kHarpMaxStages];        // floats into theta
  int64_t fallback_off[kHarpMaxStages];     // floats into fallbacks (radices not a power of two)
  int64_t blocks_off[kHarpMaxStages];       // floats into the block table
};

struct HarpArgs {
  const float* x;
  float* y;              // fp32 output or null
  int64_t rows;
  int d;
  HarpSchedule sc;
  const float* blocks;
  int inverse;
  int group;
  uint8_t* codes;        // packed int4 output or null
  void* scales;
  int scale_f16;
  int rows_per_group;    // set by the launcher
  int stream;            // set by the launcher: nontemporal row loads
};

hipError_t launch_harp_blocks(const HarpSchedule& sc, const float* theta, const float* fallbacks,
                              float* blocks, hipStream_t s);
hipError_t launch_harp_apply(HarpArgs a, hipStream_t s);

hipError_t launch_rht(const RhtArgs& a, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, hipStream_t s);
bool launch_rht2048(const RhtArgs& a, hipStream_t s);  // false: not handled
bool launch_rht2048_mfma(const RhtArgs& a, hipStream_t s);  // false: not handled
bool launch_mixed2048_mfma(const RhtArgs& a, hipStream_t s);  // false: not handled
hipError_t launch_butterfly_coeffs(const float* angles, int n, int log2n, int precondition,
                                   float* coeffs, hipStream_t s);
hipError_t launch_butterfly(const ButterflyArgs& a, hipStream_t s);
bool launch_butterfly4096(const ButterflyArgs& a, hipStream_t s);  // false: not handled
hipError_t launch_dequant(const uint8_t* codes, const void* scales, int scale_f16, int64_t rows,
                          int n, int group, float* out, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// bf16 rows of n = 2048 or 4096, int4 codes in the tiled fp6 format (a.codes)
// and transposed scales (a.scales), G = 128 or 256; false for other cases
bool launch_rotate_quant_fp6(const RhtArgs& a, hipStream_t s);
// scales may be null (then out_scales, scale_f16 and group are unused)
hipError_t launch_int4_to_fp6(const uint8_t* codes, const void* scales, bool scale_f16, int64_t rows, int64_t K,
                              int group, uint8_t* out, void* out_scales, hipStream_t s);
// a.a, a.w: tiled fp6; a.sa, a.sw: transposed scales [K / G][padded rows]
hipError_t launch_gemm_fp6(const GemmArgs& a, hipStream_t s);
hipError_t launch_rotate_quant_gemm_decode(const FusedDecodeArgs& a, hipStream_t s);
bool launch_gemm_mfma(const GemmArgs& a, hipStream_t s);  // false: not handled

}  // namespace hr
