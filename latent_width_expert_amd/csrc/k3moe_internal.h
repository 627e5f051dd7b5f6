// Internal interfaces between the C-ABI host code and the HIP kernels of the LatentMoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {

// ---------------------------------------------------------------------------------------------
// Packed weight layout ("panels").
//
// A weight matrix W[N, K] (N outputs, K reduction, MXFP4 with one E8M0 scale per 32 K) is cut
// into panels of 64 output rows; each panel is a sequence of windows of 128 K. One panel-window
// is 4352 bytes:
//   bytes [0, 4096):    4 row-tiles x 64 lanes x 16 bytes. Lane l of row-tile rt holds the 32
//                       E2M1 codes (one MX block, element 2i in the low nibble) of row
//                       16 rt + (l % 16), K block 4 w + l / 16.
//   bytes [4096, 4352): 64 lanes x 4 bytes; byte rt of lane l is the E8M0 scale of that block.
// One lane's 16 bytes are exactly the operand of one MFMA lane (16x16 tiles, K split in four
// 32-element blocks across the lane groups), and a wave reads a panel-window with five fully
// coalesced loads. Rows past N and K blocks past K are zero.
//
// GLU panels (gate and up of one GLU packed together): panel p holds hidden units
// [32 p, 32 p + 32): row-tile 0 = gate rows 32p..32p+15, 1 = up rows of the same units,
// 2 = gate rows 32p+16..32p+31, 3 = up rows of those, so SiLU(gate) * up needs no data exchange.
// ---------------------------------------------------------------------------------------------
constexpr int kPanelRows = 64;
constexpr int kWinK = 128;
constexpr int kPanelWinBytes = 4352;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct PackSrc {
  const uint8_t* codes;   // canonical [N][K/2]
  const uint8_t* scales;  // canonical [N][K/32]
  int32_t N, K;
};

struct PackJob {
  uint8_t* dst;       // first panel of the panel group
  int32_t wwin;       // windows per panel in this group
  int32_t p_off;      // first panel written by this job
  int32_t P;          // panels written by this job
  int32_t glu;        // 1: GLU panels from src[0] (gate) and src[1] (up)
  int32_t nseg;       // plain panels: K segments, src[s] covering K blocks [kb0[s], kb0[s] + K/32)
  int32_t kb0[4];
  PackSrc src[4];
};

// ---------------------------------------------------------------------------------------------
// Panel GEMM: C[rows, panels] = A[rows, K] * W^T with an epilogue chosen per panel range.
// ---------------------------------------------------------------------------------------------
enum EpiMode : int32_t {
  EPI_F32 = 0,          // fp32 out
  EPI_BF16 = 1,         // bf16 out
  EPI_SIGMOID = 2,      // fp32 sigmoid(v) out
  EPI_SWIGLU_BF16 = 3,  // GLU panels: bf16 SiLU(gate) * up
  EPI_SWIGLU_MXFP8 = 4, // GLU panels: MXFP8 of SiLU(gate) * up (blocks of 32 units)
  EPI_MXFP8 = 5,        // MXFP8 out (blocks of 32 columns)
  EPI_BF16_ADD = 6      // bf16(v + addend)
};
enum AFmt : int32_t { A_BF16 = 0, A_MXFP8 = 1 };

struct EpiSeg {
  int32_t p0, p1;         // panels [p0, p1) use this segment
  int32_t mode;           // EpiMode
  int32_t ncols;          // valid output columns (units for GLU modes) of the segment
  int32_t col0;           // column offset in `out` (and `pre`, `addend`)
  int32_t pad_;
  void* out;              // row-major, leading dimension ldo (elements)
  int64_t ldo;
  uint8_t* out_scales;    // MXFP8 modes: E8M0 bytes, leading dimension ldos
  int64_t ldos;
  float* pre;             // optional fp32 copy of the values before quantisation (ld ldpre)
  int64_t ldpre;
  const float* addend;    // EPI_BF16_ADD (ld ldadd)
  int64_t ldadd;
};
constexpr int kMaxSeg = 6;

struct GemmArgs {
  const uint8_t* W;        // packed panels of group 0
  int64_t w_group_stride;  // bytes between groups' panel sets
  int32_t P;               // panels per group
  int32_t wwin;            // windows per panel
  int32_t K;               // reduction length (multiple of 32)
  int32_t a_fmt;           // AFmt
  const void* A;           // bf16 or E4M3 codes, row-major, leading dimension lda (elements)
  int64_t lda;
  int64_t a_bytes;         // bytes of A (loads past it read zeros); below 2^31 - 2^24
  const uint8_t* A_scales; // MXFP8: E8M0 bytes, leading dimension ldas
  int64_t ldas;
  int64_t as_bytes;        // bytes of A_scales
  const int32_t* rowmap;   // optional: output row -> A row
  const int32_t* offsets;  // grouped: rows of group g are [offsets[g], offsets[g+1])
  int32_t n_groups;        // grouped: number of groups
  int32_t M;               // dense: rows; grouped: rows over every group (0: unknown)
  int32_t m_passes;        // dense: row passes (set by the launcher)
  int32_t row_split;       // grouped: 0 = the panel kernel takes every group; 1 = the row-tiled kernel takes
                           // every group; n > 1 = groups of at least n rows take the row-tiled kernel and
                           // the others the panel kernel (both launched; each skips the other's groups)
  int32_t row_cap;         // grouped, row-tiled kernel: when > 0, groups of row_cap or more rows are left to
                           // another launch; mid-row kernel: its groups have fewer (set by the launcher)
  int32_t panel_major;     // dense, row-tiled kernel: blocks dealt panel block first (set by the launcher)
  int32_t* items;          // grouped, row-tiled kernel: workspace of tile_items_bytes() for the work-item
                           // list (persistent grid); null: one block per (group, panel block)
  int32_t nseg;
  EpiSeg seg[kMaxSeg];
  float* partial;          // dense launches of few rows: split-K partial sums (workspace), may be null
  int64_t partial_bytes;   // at least gemm_partial_bytes() to be used
  // BF16 LoRA delta of a grouped stage (lora_t null: none). Output column n of group g in row `row`
  // gains sum_{q < lora_rank} lora_t[row * lora_ldt + q0 + q] * B[n * lora_ldb + q0 + q], with
  // B = lora_b + g * lora_b_stride (bf16) and q0 = lora_rank for the up units of GLU panels, else 0.
  const float* lora_t;
  int32_t lora_ldt;
  int32_t lora_rank;       // a multiple of 8
  const uint16_t* lora_b;
  int64_t lora_b_stride;   // elements between groups
  int32_t lora_ldb;        // elements per row of B
  int32_t pad2_;
};

enum GemmStage : int { GEMM_X = 0, GEMM_GATEUP = 1, GEMM_DOWN = 2, GEMM_Y = 3 };

hipError_t launch_pack(const PackJob& job, hipStream_t s);
// Grouped launches (offsets != null) use n_groups blocks along y; dense launches cover M rows.
hipError_t launch_panel_gemm(const GemmArgs& a, GemmStage stage, hipStream_t s);
// workspace for the split-K partial sums of dense launches of at most 64 rows
int64_t gemm_partial_bytes();
// workspace for the work-item list of grouped row-tiled launches: a header of kItemHeader ints
// (start of each XCD's list, then the total), then one int per item (expert | chunk << 12 |
// panel block << 24) for up to max_rows rows over n_groups groups and at most nblk panel blocks
// (chunks of at least 64 rows); tile_items_fit says whether the item format holds the launch
constexpr int kItemHeader = 16;
int64_t tile_items_bytes(int64_t max_rows, int n_groups, int nblk);
bool tile_items_fit(int64_t max_rows_per_group, int n_groups, int nblk);
hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* idx, float* p,
                       hipStream_t s);
// scratch: route_scratch_bytes(max_tokens, E) bytes of workspace (per-chunk expert counts); small T
// (or scratch == null) takes the single-block kernel
hipError_t launch_route(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv, int32_t* scratch, hipStream_t s);
int64_t route_scratch_bytes(int max_tokens, int E);
// mode 0: n = bf16(gamma * u / sqrt(mean(u^2) + eps)) into n_out (ld ldn); mode 1: u only
hipError_t launch_combine(const float* O, const int32_t* inv, const float* p, int T, int k, int width,
                          const float* gamma, float eps, int mode, uint16_t* n_out, int64_t ldn, float* u_out,
                          hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);

// LoRA first factor of a grouped stage: t[row, n] = sum_k act[row, k] La_g[n, k] over the rows of each
// group g (La bf16 [N, K] per group, la_stride elements apart, N <= 64 and a multiple of 8); the
// activation rows are bf16 or MXFP8 (codes + E8M0 scales), addressed through the optional row map.
struct LoraAArgs {
  const void* A;
  int64_t lda;
  int64_t a_bytes;
  const uint8_t* A_scales;
  int64_t ldas;
  int64_t as_bytes;
  int32_t a_fmt;
  int32_t n_groups;
  const int32_t* rowmap;
  const int32_t* offsets;
  const uint16_t* La;
  int64_t la_stride;
  int32_t N, K;
  float* t;
  int64_t ldt;
};
hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s);

// Expert-parallel send side: rows[r] = src[perm[r]] for r < n_rows (row_bytes each, a multiple of 16),
// and the MXFP8 scale rows likewise (scale_bytes each, may be 0); send_counts[i] = offsets[(i + 1) per]
// - offsets[i per] for i < n_ranks.
hipError_t launch_gather_rows(const uint8_t* src, int64_t row_bytes, const uint8_t* src_scales, int64_t scale_bytes,
                              const int32_t* perm, int64_t n_rows, uint8_t* rows, uint8_t* scales, hipStream_t s);
hipError_t launch_send_counts(const int32_t* offsets, int n_ranks, int per, int32_t* send_counts, hipStream_t s);
// offsets[0..E] = exclusive prefix sum of max(counts[e], 0), each clamped to `limit` (one block)
hipError_t launch_offsets(const int32_t* counts, int E, int64_t limit, int32_t* offsets, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16) with non-temporal 16-byte loads; the xor of every word
// read is xor-ed into *out (a measurement of the plain HBM read rate).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);

// The library's static device scratch (for callers that cannot allocate): its address on the current
// device (looked up once per device) and its size.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void** out);
// b_e = -(m-th largest of scores[:, e]) for T <= 16384 calibration tokens ([T, E] fp32 scores)
hipError_t launch_quantile_bias(const float* scores, int T, int E, int m, float* bias, hipStream_t s);

}  // namespace k3
