// HIP kernels (gfx950 / CDNA4) of the Kimi K3 LatentMoE layer forward.
//
// Method: Kimi K3 course, lesson 6 "LatentMoE", eq. 11 (layer) and eq. 13 (router).
// Number formats: MXFP4 weights (E2M1 + E8M0 per 32), bf16 or MXFP8 (E4M3 + E8M0 per 32)
// activations, fp32 accumulation.
#include "k3moe_internal.h"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

namespace k3 {

typedef uint32_t u32;
typedef uint16_t u16;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// ---------------------------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------------------------

// 2^(byte - 127) as fp32 (byte 0 -> 2^-127, a subnormal).
__device__ __forceinline__ float e8m0_f32(u32 byte) {
  return __uint_as_float(byte ? (byte << 23) : 0x00400000u);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ u32 bf16_rne(float f) {
  u32 b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// E4M3 ("fn") code of x (already divided by its block scale): round to nearest even on the
// E4M3 grid, saturate at 448, keep the sign (also of a zero result). The reference definition the
// hardware conversion in mxfp8_block is held to; the kernels call the conversion.
__device__ __forceinline__ u32 e4m3_code(float x) {
  // both ranges computed and one selected: no divergent branch per element
  const u32 sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  const u32 sub = (u32)rintf(a * 512.0f);  // subnormal grid step 2^-9; 8 steps = smallest normal (code 8)
  u32 b = __float_as_uint(a);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;  // keep 3 mantissa bits, ties to even
  b = __float_as_uint(fminf(__uint_as_float(b), 448.0f));
  const u32 nrm = ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
  return sign | (a < 0x1p-6f ? sub : nrm);
}

// E8M0 byte of an MX block with largest magnitude amax > 0 for an element format whose largest
// binade starts at 2^emax: exponent floor(log2 amax) - emax, clamped to [-127, 127].
__device__ __forceinline__ int mx_shared_exp(float amax, int emax) {
  // frexp exponent: amax = m 2^x with m in [0.5, 1), so floor(log2 amax) = x - 1 (denormals included)
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// SiLU(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about one ulp each); a gate
// below about -88 gives e^-g = inf and SiLU = -0.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Raw buffer loads: the hardware bounds-checks every load against the resource's byte count and
// returns zeros for out-of-range offsets without touching memory, so tails and masked lanes need
// no branches (and the wait counters stay exact).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kOOB = 0x7F000000;        // an offset past every resource (resources stay below it)
constexpr int kNT = 2;                  // non-temporal cache policy

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// ---------------------------------------------------------------------------------------------
// Packer: canonical MXFP4 -> panels. One thread per (panel, window, lane).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void pack_kernel(PackJob job) {
  const int lane = threadIdx.x;
  const int p = blockIdx.x;  // panel within the job
  const int w = blockIdx.y;  // window
  const int j = lane & 15, g = lane >> 4;
  const int kb = 4 * w + g;
  uint8_t* dst = job.dst + ((int64_t)(job.p_off + p) * job.wwin + w) * kPanelWinBytes;
  u32 sc_word = 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    int si = -1, n = 0, kbl = -1;
    if (job.glu) {
      si = rt & 1;
      n = 32 * p + (rt >> 1) * 16 + j;
      kbl = kb;
    } else {
      n = 64 * p + 16 * rt + j;
      for (int s = 0; s < job.nseg; ++s) {
        int nkb = job.src[s].K / 32;
        if (kb >= job.kb0[s] && kb < job.kb0[s] + nkb) {
          si = s;
          kbl = kb - job.kb0[s];
        }
      }
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    u32 sc = 0;
    if (si >= 0) {
      const PackSrc src = job.src[si];
      if (n < src.N && kbl >= 0 && kbl < src.K / 32) {
        v = *(const u32x4*)(src.codes + (int64_t)n * (src.K / 2) + (int64_t)kbl * 16);
        sc = src.scales[(int64_t)n * (src.K / 32) + kbl];
      }
    }
    *(u32x4*)(dst + rt * 1024 + lane * 16) = v;
    sc_word |= sc << (8 * rt);
  }
  *(u32*)(dst + 4096 + lane * 4) = sc_word;
}

hipError_t launch_pack(const PackJob& job, hipStream_t s) {
  if (job.P <= 0 || job.wwin <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(job.P, job.wwin), dim3(64), 0, s, job);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Panel GEMM.
//
// One wave computes one panel (64 weight rows) for MT 16-row tiles of A over its share of the
// windows. Per window it loads the 4 KB of codes and 256 B of scales of the panel (5 coalesced,
// non-temporal loads per lane: the weights are streamed once and should not displace the
// activations in L2) and the lane's 32 A values per tile, converts the E2M1 codes to bf16 with
// their E8M0 scale (v_cvt_scalef32_pk_bf16_fp4, exact) and issues 16 MT MFMA 16x16x32 bf16 (each
// weight operand is converted once and reused for the MT tiles). Loads run NBUF - 1 windows
// ahead in a register ring, so each wave keeps several KB in flight.
// MFMA lane roles: A lane (i = l % 16, g = l / 16) supplies row i, B lane (j, g) weight row j;
// both take K elements [32 (4w + g) + 8 s, +8) in MFMA step s of window w; D lane (j, g) ends
// with rows 4 g + r (r = 0..3), column j.
// KSPLIT > 1: KSPLIT waves of a block split the windows of one panel and reduce through LDS in
// a fixed tree order (deterministic).
// ---------------------------------------------------------------------------------------------
template <int AFMT>
struct AWin;
template <>
struct AWin<A_BF16> {
  u32x4 v[4];
};
template <>
struct AWin<A_MXFP8> {
  u32x4 v[2];
  u32 sc;
};

struct WWin {
  u32x4 c[4];
  u32 sc;
};

template <int AFMT, int MT>
struct WinBuf {
  WWin w;
  AWin<AFMT> a[MT];
};

template <int AFMT, int MT>
struct ATile {
  AWin<AFMT> a[MT];
};

// One panel-window of the wave's window range (window wi relative to the range start).
__device__ __forceinline__ void load_w(WWin& b, rsrc_t wr, int lane, int wi) {
  const int off = wi * kPanelWinBytes;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) b.c[rt] = __builtin_amdgcn_raw_buffer_load_b128(wr, off + rt * 1024 + lane * 16, 0, kNT);
  b.sc = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 4096 + lane * 4, 0, kNT);
}

// The lane's MX block (K block kb) of A row arow; invalid lanes and blocks past K read zeros.
template <int AFMT>
__device__ __forceinline__ void load_a(AWin<AFMT>& a, rsrc_t ar, rsrc_t asr, const GemmArgs& args, int arow,
                                       bool valid, int kb);

template <>
__device__ __forceinline__ void load_a<A_BF16>(AWin<A_BF16>& a, rsrc_t ar, rsrc_t, const GemmArgs& args, int arow,
                                               bool valid, int kb) {
  const int off = (valid && kb * 32 < args.K) ? (arow * (int)args.lda + kb * 32) * 2 : kOOB;
#pragma unroll
  for (int s = 0; s < 4; ++s) a.v[s] = __builtin_amdgcn_raw_buffer_load_b128(ar, off + 16 * s, 0, 0);
}

template <>
__device__ __forceinline__ void load_a<A_MXFP8>(AWin<A_MXFP8>& a, rsrc_t ar, rsrc_t asr, const GemmArgs& args,
                                                int arow, bool valid, int kb) {
  const bool in = valid && kb * 32 < args.K;
  const int off = in ? arow * (int)args.lda + kb * 32 : kOOB;
  a.v[0] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
  a.v[1] = __builtin_amdgcn_raw_buffer_load_b128(ar, off + 16, 0, 0);
  a.sc = __builtin_amdgcn_raw_buffer_load_b8(asr, in ? arow * (int)args.ldas + kb : kOOB, 0, 0);
}

// bf16 operand of MFMA step s (K elements 8 s .. 8 s + 7 of the lane's block)
template <int AFMT>
__device__ __forceinline__ bf16x8 a_operand(const AWin<AFMT>& a, int s);

template <>
__device__ __forceinline__ bf16x8 a_operand<A_BF16>(const AWin<A_BF16>& a, int s) {
  return __builtin_bit_cast(bf16x8, a.v[s]);
}

template <>
__device__ __forceinline__ bf16x8 a_operand<A_MXFP8>(const AWin<A_MXFP8>& a, int s) {
  const float sc = e8m0_f32(a.sc);
  const u32 d0 = a.v[s >> 1][(s & 1) * 2 + 0];
  const u32 d1 = a.v[s >> 1][(s & 1) * 2 + 1];
  u32x4 r;
  r[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false));
  r[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true));
  r[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false));
  r[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true));
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 fp4_operand(u32 d, float sc) {
  u32x4 r;
  r[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0));
  r[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1));
  r[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2));
  r[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3));
  return __builtin_bit_cast(bf16x8, r);
}

template <int AFMT, int MT>
__device__ __forceinline__ void compute_window(f32x4 (&acc)[MT][4], const WWin& w, const AWin<AFMT> (&a)[MT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[mt] = a_operand<AFMT>(a[mt], s);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16x8 wv = fp4_operand(w.c[rt][s], e8m0_f32((w.sc >> (8 * rt)) & 0xFFu));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], wv, acc[mt][rt], 0, 0, 0);
    }
  }
}

// Maximum over each 16-lane row of the wave with DPP moves (quad swaps, then half-row and row
// mirrors): every lane of the row ends with the row maximum.
// The values are magnitudes (>= 0), whose order is the order of their bit patterns as unsigned
// integers: the maximum is taken on those (no float canonicalisation, and the DPP moves fold into the
// integer max).
__device__ __forceinline__ float row16_max(float v) {
  u32 b = __float_as_uint(v);
  b = max(b, (u32)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, true));
  b = max(b, (u32)__builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xF, 0xF, true));
  b = max(b, (u32)__builtin_amdgcn_mov_dpp((int)b, 0x141, 0xF, 0xF, true));
  b = max(b, (u32)__builtin_amdgcn_mov_dpp((int)b, 0x140, 0xF, 0xF, true));
  return __uint_as_float(b);
}

// MX encode a block of 32 values held as v0 (column j) and v1 (column 16 + j) by the 16 lanes of
// one lane group; returns the E4M3 codes of v0, v1 and the E8M0 byte. All 64 lanes must call.
__device__ __forceinline__ void mxfp8_block(float v0, float v1, u32& c0, u32& c1, u32& sbyte) {
  const float amax = row16_max(__uint_as_float(max(__float_as_uint(v0) & 0x7FFFFFFFu, __float_as_uint(v1) & 0x7FFFFFFFu)));
  const int e = mx_shared_exp(amax, 8);
  sbyte = amax == 0.0f ? 0u : (u32)(e + 127);  // an all-zero block: scale byte 0, codes +-0
  const float inv = e8m0_f32((u32)(127 - e));  // 2^-e
  // E4M3 of both scaled values in one conversion (round to nearest even, subnormals kept, sign kept;
  // the clamp gives the saturation at 448, where the conversion alone would give NaN). For finite
  // inputs it equals e4m3_code bit for bit: checked on the device over every E4M3 midpoint and its
  // fp32 neighbours, 400..600 in steps of 1/8, zeros, fp32 subnormals and 16M log-uniform values.
  const u32 pk = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v0 * inv, -448.0f), 448.0f),
                                                      fminf(fmaxf(v1 * inv, -448.0f), 448.0f), 0, false);
  c0 = pk & 0xFFu;
  c1 = (pk >> 8) & 0xFFu;
}

// sum_{q < rank} t[q] b[q] in fp32, q ascending (rank a multiple of 8; t 32-byte and b 16-byte aligned):
// one output column's BF16 LoRA delta, t the row's first-factor values, b the column's row of B.
__device__ __forceinline__ float lora_dot(const float* t, const uint16_t* b, int rank) {
  float s = 0.0f;
  for (int q = 0; q < rank; q += 8) {
    const float4 t0 = *(const float4*)(t + q), t1 = *(const float4*)(t + q + 4);
    const u32x4 bb = *(const u32x4*)(b + q);
    s = fmaf(t0.x, __uint_as_float(bb[0] << 16), s);
    s = fmaf(t0.y, __uint_as_float(bb[0] & 0xFFFF0000u), s);
    s = fmaf(t0.z, __uint_as_float(bb[1] << 16), s);
    s = fmaf(t0.w, __uint_as_float(bb[1] & 0xFFFF0000u), s);
    s = fmaf(t1.x, __uint_as_float(bb[2] << 16), s);
    s = fmaf(t1.y, __uint_as_float(bb[2] & 0xFFFF0000u), s);
    s = fmaf(t1.z, __uint_as_float(bb[3] << 16), s);
    s = fmaf(t1.w, __uint_as_float(bb[3] & 0xFFFF0000u), s);
  }
  return s;
}

// LoRA deltas of one 16 x 16 output block held as acc[r] (lane rows row0 + r, r < 4, valid while below
// r1; column col of the group's B, q0 its first rank index). Uniform branch on args.lora_t outside.
__device__ __forceinline__ void lora_add(const GemmArgs& args, f32x4& acc, int grp, int row0, int r1, int col, int q0) {
  const uint16_t* b = args.lora_b + (int64_t)grp * args.lora_b_stride + (int64_t)col * args.lora_ldb + q0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + r;
    if (row < r1) acc[r] += lora_dot(args.lora_t + (int64_t)row * args.lora_ldt + q0, b, args.lora_rank);
  }
}

// Epilogue of one 16-row tile (rows mb .. mb + 15, valid below r1) of one panel of group grp.
__device__ __forceinline__ void epilogue(const GemmArgs& args, const f32x4 (&acc_in)[4], int panel, int mb, int r1,
                                         int lane, int grp, bool lora_done = false) {
  int si = 0;
  for (int s = 0; s < args.nseg; ++s)
    if (panel >= args.seg[s].p0 && panel < args.seg[s].p1) si = s;
  const EpiSeg& sg = args.seg[si];
  const int j = lane & 15, gq = lane >> 4;
  const int pl = panel - sg.p0;
  const int mode = sg.mode;
  f32x4 acc[4] = {acc_in[0], acc_in[1], acc_in[2], acc_in[3]};
  if (args.lora_t && !lora_done) {
    if (mode == EPI_SWIGLU_BF16 || mode == EPI_SWIGLU_MXFP8) {
      // row-tiles: gate and up of units 32 pl + j, then of units 32 pl + 16 + j
      const int R = args.lora_rank;
      lora_add(args, acc[0], grp, mb + 4 * gq, r1, 32 * pl + j, 0);
      lora_add(args, acc[1], grp, mb + 4 * gq, r1, 32 * pl + j, R);
      lora_add(args, acc[2], grp, mb + 4 * gq, r1, 32 * pl + 16 + j, 0);
      lora_add(args, acc[3], grp, mb + 4 * gq, r1, 32 * pl + 16 + j, R);
    } else {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int col = 64 * pl + 16 * rt + j;
        if (col < sg.ncols) lora_add(args, acc[rt], grp, mb + 4 * gq, r1, col, 0);
      }
    }
  }
  if (mode == EPI_SWIGLU_BF16 || mode == EPI_SWIGLU_MXFP8 || mode == EPI_MXFP8) {
    const bool glu = mode != EPI_MXFP8;
    const int nblk = glu ? 1 : 2;  // 32-wide blocks per panel: GLU 32 units, plain 64 columns
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb + 4 * gq + r;
      const bool ok = row < r1;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= nblk) break;  // uniform; static indices keep acc in registers
        float v0, v1;
        int c0i, c1i;  // columns of v0, v1 within the segment
        if (glu) {
          v0 = silu(acc[0][r]) * acc[1][r];  // unit 32 pl + j
          v1 = silu(acc[2][r]) * acc[3][r];  // unit 32 pl + 16 + j
          c0i = 32 * pl + j;
          c1i = 32 * pl + 16 + j;
        } else {
          v0 = acc[2 * q][r];
          v1 = acc[2 * q + 1][r];
          c0i = 64 * pl + 32 * q + j;
          c1i = 64 * pl + 32 * q + 16 + j;
        }
        if (sg.pre && ok) {
          if (c0i < sg.ncols) sg.pre[(int64_t)row * sg.ldpre + sg.col0 + c0i] = v0;
          if (c1i < sg.ncols) sg.pre[(int64_t)row * sg.ldpre + sg.col0 + c1i] = v1;
        }
        if (mode == EPI_SWIGLU_BF16) {
          if (ok) {
            u16* o = (u16*)sg.out + (int64_t)row * sg.ldo + sg.col0;
            if (c0i < sg.ncols) o[c0i] = (u16)bf16_rne(v0);
            if (c1i < sg.ncols) o[c1i] = (u16)bf16_rne(v1);
          }
        } else {
          u32 k0, k1, sb;
          mxfp8_block(v0, v1, k0, k1, sb);
          if (ok) {
            uint8_t* o = (uint8_t*)sg.out + (int64_t)row * sg.ldo + sg.col0;
            if (c0i < sg.ncols) o[c0i] = (uint8_t)k0;
            if (c1i < sg.ncols) o[c1i] = (uint8_t)k1;
            if (j == 0 && c0i < sg.ncols) sg.out_scales[(int64_t)row * sg.ldos + (sg.col0 + c0i) / 32] = (uint8_t)sb;
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int col = 64 * pl + 16 * rt + j;
    if (col >= sg.ncols) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb + 4 * gq + r;
      if (row >= r1) continue;
      const float v = acc[rt][r];
      const int64_t o = (int64_t)row * sg.ldo + sg.col0 + col;
      if (mode == EPI_F32) {
        ((float*)sg.out)[o] = v;
      } else if (mode == EPI_SIGMOID) {
        ((float*)sg.out)[o] = 1.0f / (1.0f + expf(-v));
      } else if (mode == EPI_BF16) {
        ((u16*)sg.out)[o] = (u16)bf16_rne(v);
        if (sg.pre) sg.pre[(int64_t)row * sg.ldpre + sg.col0 + col] = v;
      } else {  // EPI_BF16_ADD
        ((u16*)sg.out)[o] = (u16)bf16_rne(v + sg.addend[(int64_t)row * sg.ldadd + sg.col0 + col]);
      }
    }
  }
}

// Workgroup barrier after this wave's LDS operations have completed, without waiting for its
// outstanding global loads (a weight ring in flight stays in flight); also a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only: this wave's LDS writes and reads are done
  asm volatile("s_barrier" ::: "memory");
}

// Waves per block: KSPLIT waves per panel, 4 panels per block when KSPLIT == 1.
template <int KSPLIT>
struct BlockShape {
  static constexpr int waves = KSPLIT == 1 ? 4 : KSPLIT;
  static constexpr int panels = KSPLIT == 1 ? 4 : 1;
};

// TAG only separates the stages (x_gemm, gateup, down, y_gemm) into distinct kernel symbols.
// AHEAD: A tiles travel in the weight ring (prefetched NBUF - 1 windows ahead, few rows per
// wave); otherwise each window's A tile is loaded just before the next weight prefetch (MT
// tiles of A would not fit the ring), so waiting for it never waits for that prefetch.
// LR > 0 (grouped launches with BF16 LoRA deltas of rank at most LR): the delta of the tile is
// added to the accumulators by fp32 MFMA 16x16x4 steps before the epilogue, with lane group g
// taking rank indices [g LR/4, (g + 1) LR/4) on both operands; its operands (the tile's rows of
// t = A v and the panel's columns of B) are loaded before the window loop, so their latency hides
// behind the weight stream instead of following it.
// ASH (grouped launches of up to 16 rows per expert, several rows each): the four waves of a block (one
// expert, four panels) share the expert's 16-row A tile: each wave loads a quarter of the window's tile
// into its ring, writes it to one of two LDS stages the window it is used, and after one barrier every
// wave reads its operands from there (16-byte chunk c of row r at position c ^ r, conflict-free).
// A costs one load per lane and window instead of four, which leaves the weight stream more of the
// per-CU load path.
template <int KSPLIT, int AFMT, int NBUF, int MT, bool AHEAD, int LR, bool ASH, int TAG>
__global__ __launch_bounds__(64 * BlockShape<KSPLIT>::waves) void panel_gemm_kernel(GemmArgs args) {
  static_assert(LR == 0 || (MT == 1 && KSPLIT == 1 && LR % 16 == 0 && LR <= 32), "LoRA tiles");
  static_assert(!ASH || (MT == 1 && KSPLIT == 1 && LR == 0), "shared A tiles");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps the resources scalar
  int pblock, grp = 0, r0, r1;
  if (args.offsets) {
    pblock = blockIdx.x;
    grp = blockIdx.y;
    r0 = args.offsets[grp];
    r1 = args.offsets[grp + 1];
  } else {
    // Dense: the M passes of one panel block are placed on block ids b = 32 q + 8 m + r (pass m,
    // panel block 8 q + r). Blocks are dealt to the 8 XCDs round robin, so the passes of a panel
    // run on the same XCD one after another and re-read its weights from that XCD's L2.
    const int b = blockIdx.x;
    const int per = 8 * args.m_passes;
    const int m = (b % per) / 8;
    pblock = (b / per) * 8 + b % 8;
    r0 = m * 16 * MT;
    r1 = min(r0 + 16 * MT, args.M);
  }
  const int panel = pblock * BlockShape<KSPLIT>::panels + wave / KSPLIT;
  const int ks = wave % KSPLIT;
  const bool panel_ok = panel < args.P;
  if (r0 >= r1 || pblock * BlockShape<KSPLIT>::panels >= args.P) return;  // uniform over the block
  if (args.offsets && args.row_split > 1 && r1 - r0 >= args.row_split) return;  // the row-tiled kernel's group

  const int wbeg = (args.wwin * ks) / KSPLIT;
  const int wend = (args.wwin * (ks + 1)) / KSPLIT;
  // with a shared A tile every wave of the block runs every window (the barriers), a wave past the
  // last panel on a weight resource of no bytes
  const int nwin = (ASH || panel_ok) ? wend - wbeg : 0;
  const rsrc_t wr = make_rsrc(args.W + (int64_t)grp * args.w_group_stride +
                                  ((int64_t)(panel_ok ? panel : 0) * args.wwin + wbeg) * kPanelWinBytes,
                              (int64_t)(panel_ok ? nwin : 0) * kPanelWinBytes);
  const rsrc_t ar = make_rsrc(args.A, args.a_bytes);
  const rsrc_t asr = make_rsrc(args.A_scales, args.A_scales ? args.as_bytes : 0);
  const int g = lane >> 4;

  // partial sums of the upper half of the K-split waves, per tree level
  __shared__ f32x4 red[KSPLIT > 1 ? (KSPLIT / 2) * MT * 4 * 64 : 1];
  // shared A tile stages: bf16 16 rows x 256 bytes; MXFP8 16 rows x 128 bytes of codes + 16 scale words
  constexpr int ASTG = AFMT == A_BF16 ? 4096 : 2048 + 64;
  __shared__ __attribute__((aligned(16))) uint8_t ash[ASH ? 2 : 1][ASH ? ASTG : 16];

  for (int mb = r0; mb < r1; mb += 16 * MT) {
    bool rv[MT];
    int arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = mb + 16 * mt + (lane & 15);
      rv[mt] = row < r1;
      arow[mt] = rv[mt] ? (args.rowmap ? args.rowmap[row] : row) : 0;
    }

    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LoRA operands of this tile (LR > 0): lt[qg][s] = t[row][qg rank + g LS + s] for the lane's A
    // row (qg 1: the up half of a GLU's t), lb[ct][s] = B[col][q0 + g LS + s] for the lane's column
    // of row-tile ct (bf16 pairs); lane groups past the rank hold zeros.
    constexpr int LS = LR > 0 ? LR / 4 : 2;
    constexpr bool GLU = TAG == GEMM_GATEUP;
    [[maybe_unused]] f32x4 lt[2][LS / 4 > 0 ? LS / 4 : 1];
    [[maybe_unused]] u32 lb[4][LS / 2];
    auto lora_loads = [&]() {
      if constexpr (LR > 0) {
        const int rank = args.lora_rank;
        const bool gok = (g + 1) * LS <= rank;
        const int row = mb + (lane & 15);
#pragma unroll
        for (int qg = 0; qg < 2; ++qg)
#pragma unroll
          for (int v = 0; v < LS / 4; ++v) lt[qg][v] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gok && row < r1) {
          const float* tp = args.lora_t + (int64_t)row * args.lora_ldt + g * LS;
#pragma unroll
          for (int qg = 0; qg < (GLU ? 2 : 1); ++qg)
#pragma unroll
            for (int v = 0; v < LS / 4; ++v) lt[qg][v] = *(const f32x4*)(tp + qg * rank + 4 * v);
        }
        const int j = lane & 15;
        const uint16_t* bb = args.lora_b + (int64_t)grp * args.lora_b_stride + g * LS;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int col = GLU ? 32 * panel + 16 * (ct >> 1) + j : 64 * panel + 16 * ct + j;
          const int q0 = GLU && (ct & 1) ? rank : 0;
          const bool ok = gok && panel_ok && col < args.seg[0].ncols;
#pragma unroll
          for (int v = 0; v < LS / 2; ++v) lb[ct][v] = 0u;
          if (ok) {
            const uint16_t* bp = bb + (int64_t)col * args.lora_ldb + q0;
            if constexpr (LS == 4) {
              const uint2 w2 = *(const uint2*)bp;
              lb[ct][0] = w2.x;
              lb[ct][1] = w2.y;
            } else {
              static_assert(LS == 8, "rank classes 16 and 32");
              const u32x4 w4 = *(const u32x4*)bp;
#pragma unroll
              for (int v = 0; v < 4; ++v) lb[ct][v] = w4[v];
            }
          }
        }
      }
    };
    auto lora_mfma = [&]() {
      if constexpr (LR > 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int qg = GLU ? (ct & 1) : 0;
#pragma unroll
          for (int st = 0; st < LS; ++st) {
            const u32 w = lb[ct][st / 2];
            const float bv = __uint_as_float(st % 2 ? (w & 0xFFFF0000u) : (w << 16));
            acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(lt[qg][st / 4][st % 4], bv, acc[0][ct], 0, 0, 0);
          }
        }
      }
    };

    // Loads are issued unconditionally: past the range they return zeros without memory traffic.
    auto load_tile = [&](AWin<AFMT>(&at)[MT], int wi) {
      const int kb = wi < nwin ? 4 * (wbeg + wi) + g : (1 << 24);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) load_a<AFMT>(at[mt], ar, asr, args, arow[mt], rv[mt], kb);
    };
    if constexpr (ASH) {
      // this lane's piece of the block's tile: bf16, 16-byte chunk pc of row pr (256 pieces, every lane
      // of the 4 waves); MXFP8, chunk pc of row pr for the 128 lanes of waves 0 and 1, and the row's
      // scale word (4 K blocks) for lanes 0..15 of wave 2
      const int pi = 64 * wave + lane;
      const int pr = AFMT == A_BF16 ? pi >> 4 : (wave < 2 ? pi >> 3 : (wave == 2 ? lane : 16));
      const int pc = AFMT == A_BF16 ? pi & 15 : pi & 7;
      const bool pv = pr < 16 && mb + pr < r1 && (AFMT == A_BF16 || wave < 2 || (wave == 2 && lane < 16));
      const int parow = pv ? (args.rowmap ? args.rowmap[mb + pr] : mb + pr) : 0;
      struct SBuf {
        WWin w;
        u32x4 p;
      };
      // pieces past K (a K tail inside the last window) read zeros, like the per-wave loads
      auto load_piece = [&](SBuf& b, int wi) {
        const bool in = pv && wi < nwin;
        const int k0 = kWinK * (wbeg + wi);  // first K element of the window
        if constexpr (AFMT == A_BF16) {
          const int off = in && k0 + 8 * pc < args.K ? (parow * (int)args.lda + k0 + 8 * pc) * 2 : kOOB;
          b.p = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        } else if (wave < 2) {
          const int off = in && k0 + 16 * pc < args.K ? parow * (int)args.lda + k0 + 16 * pc : kOOB;
          b.p = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        } else {
          u32 w = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kb = k0 / 32 + q;
            w |= (u32)__builtin_amdgcn_raw_buffer_load_b8(asr, in && 32 * kb < args.K ? parow * (int)args.ldas + kb : kOOB,
                                                          0, 0) << (8 * q);
          }
          b.p = u32x4{w, 0u, 0u, 0u};
        }
      };
      auto store_piece = [&](const SBuf& b, int stage) {
        uint8_t* st = &ash[stage][0];
        if constexpr (AFMT == A_BF16) {
          *(u32x4*)(st + 256 * pr + 16 * (pc ^ pr)) = b.p;
        } else if (wave < 2) {
          *(u32x4*)(st + 128 * pr + 16 * (pc ^ (pr & 7))) = b.p;
        } else if (wave == 2 && lane < 16) {
          *(u32*)(st + 2048 + 4 * pr) = b.p[0];
        }
      };
      auto read_tile = [&](AWin<AFMT>& at, int stage) {
        const uint8_t* st = &ash[stage][0];
        const int i16 = lane & 15;
        if constexpr (AFMT == A_BF16) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) at.v[s2] = *(const u32x4*)(st + 256 * i16 + 16 * ((4 * g + s2) ^ i16));
        } else {
          at.v[0] = *(const u32x4*)(st + 128 * i16 + 16 * ((2 * g) ^ (i16 & 7)));
          at.v[1] = *(const u32x4*)(st + 128 * i16 + 16 * ((2 * g + 1) ^ (i16 & 7)));
          at.sc = st[2048 + 4 * i16 + g];
        }
      };
      SBuf buf[NBUF];
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i) {
        load_w(buf[i].w, wr, lane, i);
        load_piece(buf[i], i);
      }
      for (int w0 = 0; w0 < nwin; w0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          SBuf& nb = buf[(u + NBUF - 1) % NBUF];
          load_w(nb.w, wr, lane, w0 + u + NBUF - 1);
          load_piece(nb, w0 + u + NBUF - 1);
          if (w0 + u < nwin) {  // uniform over the block
            // stage (w & 1) was last read in window w - 2, before every wave reached the barrier of w - 1
            store_piece(buf[u], (w0 + u) & 1);
            lds_barrier();
            AWin<AFMT> at[1];
            read_tile(at[0], (w0 + u) & 1);
            compute_window<AFMT, 1>(acc, buf[u].w, at);
          }
        }
      }
    } else if constexpr (AHEAD) {
      WinBuf<AFMT, MT> buf[NBUF];
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i) {
        load_w(buf[i].w, wr, lane, i);
        load_tile(buf[i].a, i);
      }
      lora_loads();
      for (int w0 = 0; w0 < nwin; w0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          WinBuf<AFMT, MT>& nb = buf[(u + NBUF - 1) % NBUF];
          load_w(nb.w, wr, lane, w0 + u + NBUF - 1);
          load_tile(nb.a, w0 + u + NBUF - 1);
          if (w0 + u < nwin) compute_window<AFMT, MT>(acc, buf[u].w, buf[u].a);
        }
      }
    } else {
      WWin wb[NBUF];
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i) load_w(wb[i], wr, lane, i);
      lora_loads();
      for (int w0 = 0; w0 < nwin; w0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          ATile<AFMT, MT> at;
          load_tile(at.a, w0 + u);
          load_w(wb[(u + NBUF - 1) % NBUF], wr, lane, w0 + u + NBUF - 1);
          if (w0 + u < nwin) compute_window<AFMT, MT>(acc, wb[u], at.a);
        }
      }
    }

    if constexpr (KSPLIT > 1) {
      // tree: at each level the upper half of the active waves hands its sums to the lower half
#pragma unroll
      for (int half = KSPLIT / 2; half >= 1; half >>= 1) {
        if (ks >= half && ks < 2 * half) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) red[(((ks - half) * MT + mt) * 4 + rt) * 64 + lane] = acc[mt][rt];
        }
        __syncthreads();
        if (ks < half) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[mt][rt] += red[((ks * MT + mt) * 4 + rt) * 64 + lane];
        }
        __syncthreads();
      }
    }
    lora_mfma();
    if (panel_ok && ks == 0) {
      for (int mt = 0; mt < MT && mb + 16 * mt < r1; ++mt) {
        // copy tile mt out with static indices (the loop itself stays rolled)
        f32x4 tile[4];
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
          if (m2 == mt) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) tile[rt] = acc[m2][rt];
          }
        epilogue(args, tile, panel, mb + 16 * mt, r1, lane, grp, LR > 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Scaled MFMA operands and LDS-DMA helpers (used by the row-tiled kernel below).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes E4M3 A and E2M1 B with their E8M0 block scales and
// accumulates in fp32, so neither operand is converted. Operand lanes (gfx950, established on
// the device): fp8 A lane (i = l % 16, g = l / 16) holds row i, K bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) of the 128-wide window; fp4 B lane (j, g) holds weight row j, K
// [32 g, 32 g + 32) -- exactly one lane's 16 bytes of a packed panel-window; the scale operand of
// lane (r, g) is the scale of row r, K block g (a byte of a 32-bit register chosen by opsel).
// ---------------------------------------------------------------------------------------------
typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));


// LDS-DMA (buffer_load ... lds) of 16 / 4 bytes per lane: lane l's data lands at LDS address
// lds + 16 l / lds + 4 l. Issued from asm, so the compiler neither orders its own LDS reads behind
// these writes (the kernel's explicit vmcnt wait and barrier order them) nor reuses M0 across
// them (M0, which holds the LDS address, is saved and restored). The resource is four SGPRs:
// base, stride 0, byte count, raw-buffer word 3. NT: non-temporal (streamed weights); otherwise
// the default policy (activation rows stay in L2 for the other panel blocks of the group).
typedef int i32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4s sgpr_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  i32x4s r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kRsrcWord3;
  return r;
}
__device__ __forceinline__ u32 lds_addr(const void* p) {
  return (u32)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// The DMA operands that must sit in scalar registers (the buffer resource and the LDS address, which
// are uniform over the wave by construction) pass through readfirstlane, a no-op for values the
// compiler already keeps scalar and a guarantee where it cannot prove them uniform.
__device__ __forceinline__ i32x4s sgpr4(i32x4s r) {
  return i32x4s{__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}
template <bool NT>
__device__ __forceinline__ void dma16(i32x4s r, u32 lds, int voff) {
  r = sgpr4(r);
  lds = __builtin_amdgcn_readfirstlane(lds);
  int m0save;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
}
template <bool NT>
__device__ __forceinline__ void dma4(i32x4s r, u32 lds, int voff) {
  r = sgpr4(r);
  lds = __builtin_amdgcn_readfirstlane(lds);
  int m0save;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that is also a compiler memory barrier, without the cache waits of
// __syncthreads (no memory operation moves across it; the caller's explicit waits order the DMAs).
__device__ __forceinline__ void barrier_nowait() { asm volatile("s_barrier" ::: "memory"); }

// Row-tiled GEMM for many rows per weight set (prefill): MXFP4 weights against MXFP8 activations on
// the scaled MFMA (grouped: the experts' dispatched rows) or bf16 activations on the bf16 MFMA with
// the weights converted to bf16 once per window (dense: x and the latent/shared rows, in chunks of
// ROWS rows that play the part of groups).
// Block: 4 WPS waves on one group and 4 consecutive panels, WPS waves per SIMD. Wave (pm, h)
// computes panel panel0 + pm on the row tiles h, h + WPS, ... of a chunk of up to ROWS of the
// group's rows (4 column tiles of 16x16 per row tile, fp32 accumulators); with two waves per SIMD
// one wave's MFMAs run while the other waits on LDS or on its DMA issues. Per K window of 128, by
// LDS-DMA (buffer_load ... lds) issued from asm:
//   - the chunk's activation rows (MXFP8: E4M3 codes and E8M0 scales) into an A stage shared by all
//     waves, DA windows ahead (16-byte chunk c of row r stored at position c ^ (r mod CPR), CPR the
//     row's chunks: the 16 rows of a tile read one chunk each from 16 different bank groups);
//   - each panel-window of weights into a B stage, DB windows ahead, non-temporal (the weights
//     come from HBM, the activation rows mostly from L2).
// Nothing in the loop is a compiler-visible global load: one explicit vmcnt wait and a barrier per
// window order the DMAs, and the operands are plain LDS reads that the compiler places straight
// into the MFMA operand registers.
// Blocks are dealt to the XCDs so that every panel block of a group runs on the XCD of that group
// (group g on XCD g mod 8): the group's activation rows are fetched into one L2 and re-read there.
// EPI 0: fp32 out. EPI 1: GLU panels, SiLU(gate) * up MX-encoded (E4M3, E8M0 per 32 units),
// staged in LDS and written as 16-byte row segments. EPI 2: the per-panel segment epilogues.
template <int AF, bool DENSE, int DA, int DB, int MT, int WPS, int PPW, int EPI, int TAG>
__global__ __launch_bounds__(256 * WPS) void tiled_gemm_kernel(GemmArgs args) {
  constexpr bool MX = AF == A_MXFP8;
  constexpr int NWAVE = 4 * WPS;                // WPS waves per SIMD
  constexpr int ROWS = 16 * MT, NA = DA + 1, NB = DB + 1;
  constexpr int NPG = 4 / PPW;                  // panel groups (PPW panels each)
  constexpr int NPH = NWAVE / NPG;              // row-tile phases
  constexpr int MTW = MT / NPH;                 // row tiles per wave
  constexpr int AROW = MX ? 128 : 256;          // bytes of a row's K window
  constexpr int CPR = AROW / 16;                // 16-byte chunks per row
  constexpr int SWZ = CPR - 1;                  // row bits of the chunk swizzle
  constexpr int RPD = 1024 / AROW;              // rows per 1 KB code DMA
  constexpr int ESZ = MX ? 1 : 2;               // bytes per activation element
  constexpr int A_SC = ROWS * AROW;
  constexpr int A_STAGE = A_SC + (MX ? ROWS * 4 : 0);  // MXFP8: 4 scale bytes per row (one word a K block)
  constexpr int B_STAGE = 4 * kPanelWinBytes;   // one panel-window per panel
  constexpr int APW = ROWS / RPD / NWAVE;       // 1 KB code DMAs per wave and window
  constexpr int AL = APW + (MX ? 1 : 0);        // + the wave's scale DMA
  constexpr int BPW = (20 + NWAVE - 1) / NWAVE; // the four panels' 5 weight DMAs each, over the waves
  constexpr int LPW = AL + BPW;
  static_assert(4 % PPW == 0 && MT % NPH == 0 && (ROWS / RPD) % NWAVE == 0 && (!MX || (ROWS <= 64 * NWAVE && ROWS % 64 == 0)),
                "shape");
  static_assert(DA >= 1 && DB >= 1, "ring depths");
  // At step w the later of A(w) and B(w) must have landed. DB > DA: A(w) is the later one, followed
  // by the B DMAs of its step and DA - 1 full steps; DB <= DA: B(w) comes last in its step,
  // followed by DB - 1 full steps.
  constexpr int WAITN = DB > DA ? BPW + (DA - 1) * LPW : (DB - 1) * LPW;
  static_assert(WAITN < 64, "vmcnt range");
  static_assert(EPI != 1 || (MX && ROWS * 132 <= A_STAGE), "epilogue staging fits one A stage");
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[NA][A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[NB][B_STAGE];
  // target of placeholder DMAs (zeros or unused words, never read): one 256-byte row shared by the waves
  __shared__ __attribute__((aligned(16))) uint8_t lds_sink[256];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pg = wv % NPG, h = wv / NPG;        // panel group of the wave, its row-tile phase
  const int nblk = (args.P + 3) / 4;
  // a group: an expert's rows (grouped) or a chunk of ROWS rows (dense, all on the same weights)
  const int ngrp = DENSE ? (args.M + ROWS - 1) / ROWS : args.n_groups;
  const i32x4s ar = sgpr_rsrc(args.A, args.a_bytes);
  const i32x4s asr = sgpr_rsrc(args.A_scales, MX ? args.as_bytes : 0);
  const int g = lane >> 4, i16 = lane & 15;
  const u32 lds_a0 = lds_addr(&lds_a[0][0]), lds_b0 = lds_addr(&lds_b[0][0]);
  const u32 lds_s = lds_addr(&lds_sink[0]);
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  // Work units. Grouped launches with an item list: a persistent grid (a multiple of 8 blocks) whose
  // blocks walk the run of their XCD, one item (expert, chunk of ROWS rows, panel block) at a time
  // (tile_items_kernel: equal contiguous runs, so an expert's rows and weights stay in one or two
  // XCDs' L2). Otherwise one block per (group, panel block): eight groups or more, group g on
  // XCD g mod 8; fewer, the panel blocks of each group dealt over all XCDs (block b: group b / nblk).
  const bool listed = !DENSE && args.items != nullptr;
  int it = 0, it_end = 0, it_step = 1;
  int cgrp = 0, cpanel0 = 0, cmb = 0, cr1 = 0;  // without a list: the block's group and its next chunk
  if (listed) {
    it = args.items[xcd] + slot;
    it_end = args.items[xcd + 1];
    it_step = (int)gridDim.x / 8;
  } else if (DENSE && args.panel_major) {
    // few row chunks: panel block p on XCD p mod 8 with every chunk of it side by side there, so each
    // weight panel is streamed from HBM once and the chunks re-read it from that L2 (the activation
    // rows, a few MB, are what every XCD reads)
    cpanel0 = 4 * (xcd + 8 * (slot / ngrp));
    cgrp = slot % ngrp;
    if (cpanel0 >= args.P) return;
    cmb = cgrp * ROWS;
    cr1 = min(cmb + ROWS, args.M);
  } else {
    const bool spread = ngrp < 8;
    cgrp = spread ? (int)blockIdx.x / nblk : xcd + 8 * (slot / nblk);
    cpanel0 = 4 * (spread ? (int)blockIdx.x % nblk : slot % nblk);
    if (cgrp >= ngrp) return;
    cmb = DENSE ? cgrp * ROWS : args.offsets[cgrp];
    cr1 = DENSE ? min(cmb + ROWS, args.M) : args.offsets[cgrp + 1];
    if (cmb >= cr1) return;  // uniform over the block
    // a group of another launch (the panel kernel's, or the other row band's)
    if (!DENSE && (cr1 - cmb < args.row_split || (args.row_cap > 0 && cr1 - cmb >= args.row_cap))) return;
  }
  const int nwin = args.wwin;
  const u32 a_w = lds_a0 + 1024 * (wv * APW), a_s = lds_a0 + A_SC + 256 * wv;
  // The unit in hand: rows [mb, min(mb + ROWS, r1)) of group grp (a listed item, or the next chunk of
  // the block's group) on panels panel0 .. panel0 + npan - 1, and the sources of its DMAs.
  int grp = 0, panel0 = 0, mb = 0, r1 = 0, npan = 0;
  i32x4s wr = {};
  int acode[APW], ascale = -1, akel[APW];
  auto next_unit = [&]() __attribute__((always_inline)) -> bool {
    if (listed) {
      if (it >= it_end) return false;
      const u32 item = (u32)args.items[kItemHeader + it];
      it += it_step;
      grp = (int)(item & 0xFFFu);
      panel0 = 4 * (int)(item >> 24);
      mb = args.offsets[grp] + ROWS * (int)((item >> 12) & 0xFFFu);
      r1 = min(mb + ROWS, args.offsets[grp + 1]);
    } else {
      if (cmb >= cr1) return false;
      grp = cgrp;
      panel0 = cpanel0;
      mb = cmb;
      r1 = cr1;
      cmb += ROWS;
    }
    // uniform over the block: kept in scalar registers across units
    grp = __builtin_amdgcn_readfirstlane(grp);
    panel0 = __builtin_amdgcn_readfirstlane(panel0);
    mb = __builtin_amdgcn_readfirstlane(mb);
    r1 = __builtin_amdgcn_readfirstlane(r1);
    npan = min(4, args.P - panel0);
    // the unit's (up to) four panels, one resource: panel p's window w at (p nwin + w) 4352
    wr = sgpr_rsrc(args.W + (DENSE ? 0 : (int64_t)grp * args.w_group_stride) + (int64_t)panel0 * nwin * kPanelWinBytes,
                   (int64_t)npan * nwin * kPanelWinBytes);
      // A DMAs of this wave: code instruction j = wv APW + jj covers chunk rows RPD j .. RPD j + RPD - 1
      // (lane L: row RPD j + L / CPR, position L % CPR holding 16-byte chunk (L % CPR) ^ (row & SWZ) of
      // the row's window); MXFP8: the scale instruction covers rows 64 wv .. 64 wv + 63 (lane L: row
      // 64 wv + L; waves past the chunk's rows send theirs to the sink). Elements past K read zeros;
      // rows past the chunk read zeros, or stale data where a whole piece lies past it (the rows of an
      // MFMA tile are independent, and those rows' outputs are never stored).
      #pragma unroll
      for (int jj = 0; jj < APW; ++jj) {
        const int row = mb + RPD * (wv * APW + jj) + lane / CPR;
        acode[jj] = args.rowmap ? args.rowmap[min(row, r1 - 1)] : row;
      }
      if constexpr (MX) {
        const int row = mb + 64 * wv + lane;
        ascale = args.rowmap ? args.rowmap[min(row, r1 - 1)] : row;
      }
      #pragma unroll
      for (int jj = 0; jj < APW; ++jj) {
        const int r = RPD * (wv * APW + jj) + lane / CPR;
        const int c = (lane % CPR) ^ (r & SWZ);
        akel[jj] = 16 * c / ESZ;  // first K element of the chunk inside the window
        acode[jj] = mb + r < r1 ? acode[jj] * (int)args.lda * ESZ + 16 * c : -1;
      }
      if constexpr (MX) ascale = 64 * wv + lane < ROWS && mb + 64 * wv + lane < r1 ? ascale * (int)args.ldas : -1;
    return true;
  };
      // The LPW DMAs of step w, one by one: the wave's A code DMAs, its A scale DMA, then its share
      // of the four panels' weight DMAs (items wv BPW .. wv BPW + BPW - 1 of: per panel four 1 KB code
      // pieces and the 256-byte scale piece; items past 20 are 4-byte dummies into the sink),
      // always in this order so that one wait count holds at every step. Step w fills A stage
      // (w + DA) % NA and B stage (w + DB) % NB; a window index below zero (prologue) is a dummy.
      auto issue_one = [&]<int d>(int w) {
        if constexpr (d < AL) {
          const int wa = w + DA;
          const bool real = wa >= 0;
          const bool in = real && wa < nwin;
          const u32 st = (u32)((wa % NA) * A_STAGE);
          if (!real)
            dma4<false>(ar, lds_s, kOOB);  // prologue placeholder (4 bytes a lane: the sink holds 256)
          else if constexpr (d < APW) {
            // grouped: a piece wholly past the chunk's rows becomes a 4-byte dummy into the sink (the
            // count of DMAs per step stays fixed; its stage rows keep older data, which only rows past
            // the chunk read). Dense chunks are full but for the last, and the test costs them more.
            if (!DENSE && mb + RPD * (wv * APW + d) >= r1)  // uniform
              dma4<false>(ar, lds_s, kOOB);
            else
              dma16<false>(ar, a_w + st + 1024 * d,
                           in && acode[d] >= 0 && kWinK * wa + akel[d] < args.K ? acode[d] + AROW * wa : kOOB);
          }
          else
            dma4<false>(asr, 64 * wv < ROWS ? a_s + st : lds_s, in && ascale >= 0 ? ascale + 4 * wa : kOOB);
        } else {
          const int wb = w + DB;
          const bool real = wb >= 0;
          const int item = wv * BPW + (d - AL);  // uniform
          const int p = item / 5, piece = item % 5;
          const bool in = wb < nwin && p < npan;
          const u32 st = lds_b0 + (u32)(((real ? wb : 0) % NB) * B_STAGE + p * kPanelWinBytes);
          const int src = (p * nwin + wb) * kPanelWinBytes;
          if (item >= 20 || !real)
            dma4<false>(wr, lds_s, kOOB);
          else if (piece < 4)
            dma16<true>(wr, st + 1024 * piece, in ? src + 1024 * piece + lane * 16 : kOOB);
          else
            dma4<true>(wr, st + 4096, in ? src + 4096 + lane * 4 : kOOB);
        }
      };
      auto issue_range = [&]<int D0, int D1>(int w) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (issue_one.template operator()<D0 + I>(w), ...);
        }(std::make_integer_sequence<int, D1 - D0>{});
      };
  auto prologue = [&]() __attribute__((always_inline)) {  // steps -max(DA, DB) .. -1, in steady-state order
    for (int i = -(DA > DB ? DA : DB); i < 0; ++i) issue_range.template operator()<0, LPW>(i);
  };
  f32x4 acc[MTW][PPW][4];
  // the epilogue of a unit (its rows, group end and panels given; the accumulators as they stand)
  auto finish = [&](const int mb, const int r1, const int panel0, const int npan, const int grp)
                    __attribute__((always_inline)) {
      // epilogue; lane indices re-derived (opaque to the compiler) so that no address arithmetic is
      // hoisted out of the chunk loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int eg = ln >> 4, ej = ln & 15;
      const EpiSeg& sg = args.seg[0];
      const int nrow = min(ROWS, r1 - mb);
      // BF16 LoRA deltas (grouped stages), added to the accumulators before the epilogue proper; the
      // segment epilogue (EPI 2) adds them itself
      if constexpr (EPI != 2 && !DENSE) {
        if (args.lora_t) {
          #pragma unroll
          for (int j = 0; j < MTW; ++j)
            #pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
              const int pl = PPW * pg + pp;
              const int row0 = mb + 16 * (h + NPH * j) + 4 * eg;
              if (pl < npan && row0 < r1) {
                #pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                  // EPI 1 (GLU panels): row-tiles gate / up of units 32 p + ej, then of 32 p + 16 + ej
                  const int col = EPI == 1 ? 32 * (panel0 + pl) + 16 * (ct >> 1) + ej : 64 * (panel0 + pl) + 16 * ct + ej;
                  const int q0 = EPI == 1 && (ct & 1) ? args.lora_rank : 0;
                  if (EPI == 1 || col < sg.ncols) lora_add(args, acc[j][pp][ct], grp, row0, r1, col, q0);
                }
              }
            }
        }
      }
      if constexpr (EPI == 1) {
        // codes staged as [ROWS][128 bytes] (32 units per panel), scales as [ROWS][4]
        uint8_t* stg = &lds_a[NA - 1][0];  // A stage NA - 1: no prologue DMA writes it
        uint8_t* stg_sc = stg + ROWS * 128;
        const bool tap = sg.pre != nullptr;
        const rsrc_t prr = make_rsrc(tap ? sg.pre + (int64_t)mb * sg.ldpre : nullptr,
                                     tap ? (int64_t)nrow * sg.ldpre * 4 : 0);
        #pragma unroll
        for (int j = 0; j < MTW; ++j) {
          #pragma unroll
          for (int pp = 0; pp < PPW; ++pp) {
            const int pl = PPW * pg + pp;  // panel inside the block
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v0 = silu(acc[j][pp][0][r]) * acc[j][pp][1][r];
              const float v1 = silu(acc[j][pp][2][r]) * acc[j][pp][3][r];
              const int lr = 16 * (h + NPH * j) + 4 * eg + r;
              if (tap) {
                const int o = lr * (int)sg.ldpre + sg.col0 + 32 * (panel0 + pl) + ej;
                const bool ok = lr < nrow && pl < npan;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), prr, ok ? 4 * o : kOOB, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), prr, ok ? 4 * (o + 16) : kOOB, 0, 0);
              }
              u32 c0, c1, sb;
              mxfp8_block(v0, v1, c0, c1, sb);
              stg[lr * 128 + 32 * pl + ej] = (uint8_t)c0;
              stg[lr * 128 + 32 * pl + 16 + ej] = (uint8_t)c1;
              stg_sc[lr * 4 + pl] = (uint8_t)sb;  // the 16 lanes of the block agree
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        const int t = threadIdx.x;
        uint8_t* out = (uint8_t*)sg.out + sg.col0 + 32 * panel0;
        #pragma unroll
        for (int q = 0; q < ROWS / (32 * WPS); ++q) {
          const int lr = 32 * WPS * q + t / 8, piece = t % 8;
          if (lr < nrow && piece < 2 * npan)
            *(u32x4*)(out + (int64_t)(mb + lr) * sg.ldo + 16 * piece) = *(const u32x4*)(stg + lr * 128 + 16 * piece);
        }
        for (int lr = t; lr < nrow; lr += 256 * WPS) {
          uint8_t* os = sg.out_scales + (int64_t)(mb + lr) * sg.ldos + sg.col0 / 32 + panel0;
          if (npan == 4)
            *(u32*)os = *(const u32*)(stg_sc + 4 * lr);
          else
            for (int p = 0; p < npan; ++p) os[p] = stg_sc[4 * lr + p];
        }
      } else if constexpr (EPI == 2) {
        // per-panel segment modes (sigmoid, bf16, MX encode, SwiGLU, bf16 + addend); tile and panel
        // indices are compile-time (a fold, not a loop the compiler may keep rolled), so the
        // accumulators stay in registers instead of being copied to scratch for dynamic indexing
        [&]<int... JP>(std::integer_sequence<int, JP...>) {
          ([&] {
            constexpr int j = JP / PPW, pp = JP % PPW;
            if (PPW * pg + pp < npan && 16 * (h + NPH * j) < nrow)
              epilogue(args, acc[j][pp], panel0 + PPW * pg + pp, mb + 16 * (h + NPH * j), r1, ln, grp);
          }(), ...);
        }(std::make_integer_sequence<int, MTW * PPW>{});
      } else {
        const rsrc_t orr = make_rsrc((float*)sg.out + (int64_t)mb * sg.ldo + sg.col0, (int64_t)nrow * sg.ldo * 4);
        #pragma unroll
        for (int j = 0; j < MTW; ++j) {
          #pragma unroll
          for (int pp = 0; pp < PPW; ++pp) {
            #pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
              const int pl = PPW * pg + pp;
              const int col = 64 * (panel0 + pl) + 16 * ct + ej;
              #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int lr = 16 * (h + NPH * j) + 4 * eg + r;
                const bool ok = lr < nrow && pl < npan && col < sg.ncols;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][pp][ct][r]), orr,
                                                      ok ? 4 * (lr * (int)sg.ldo + col) : kOOB, 0, 0);
              }
            }
          }
        }
      }
  };

  bool have = next_unit();
  if (have) prologue();
  while (have) {
      // row tiles holding rows (uniform over the block) and this wave's share: tiles h, h + NPH, ...
      const int nt = min(MT, (r1 - mb + 15) / 16);
      const int nw = nt > h ? (nt - h + NPH - 1) / NPH : 0;

      #pragma unroll
      for (int j = 0; j < MTW; ++j)
        #pragma unroll
        for (int pp = 0; pp < PPW; ++pp)
          #pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[j][pp][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

      // The window loop, specialised on the wave's number of row tiles holding rows (one variant per
      // count, chosen once per chunk) so that each window's body is straight-line code.
      auto run = [&]<int N>() {
        for (int w = 0; w < nwin; ++w) {
          wait_vmcnt<WAITN>();
          barrier_nowait();  // stages of w complete for every wave; stages of w - 1 free
          // weights of the wave's panel-windows
          u32x4 bw[PPW][4];
          u32 bsc[PPW];
          #pragma unroll
          for (int pp = 0; pp < PPW; ++pp) {
            const uint8_t* sb = &lds_b[w % NB][(PPW * pg + pp) * kPanelWinBytes];
            #pragma unroll
            for (int rt = 0; rt < 4; ++rt) bw[pp][rt] = *(const u32x4*)(sb + rt * 1024 + lane * 16);
            bsc[pp] = *(const u32*)(sb + 4096 + lane * 4);
          }
          // A operands: row tile t of the stage starts at t * 16 AROW (MXFP8 scales at A_SC + t * 64);
          // the swizzle depends on the row only through row % 8 = i16 % 8. MXFP8 lane (i16, g): K bytes
          // [16 g, +16) and [64 + 16 g, +16); bf16 lane (i16, g), MFMA step s: K elements [32 g + 8 s, +8).
          const uint8_t* sa = lds_a[w % NA];
          const uint8_t* prow = sa + i16 * AROW + h * 16 * AROW;
          const uint8_t* psc = sa + A_SC + i16 * 4 + g + h * 64;
          auto load_tile = [&](int j, i32x8& aop, int& asc) {  // MXFP8: the wave's j-th tile, row tile h + NPH j
            const uint8_t* pr = prow + j * NPH * 16 * AROW;
            const u32x4 lo = *(const u32x4*)(pr + 16 * (g ^ (i16 & SWZ)));
            const u32x4 hi = *(const u32x4*)(pr + 16 * ((4 + g) ^ (i16 & SWZ)));
            asc = psc[j * NPH * 64];
            aop = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          };
          // the step's DMAs are spread over the MFMA groups (the wave keeps the matrix core busy while
          // the memory pipeline drains); the next group's operands are read before each group of
          // DMAs, which are compiler barriers for memory operations
          if constexpr (N == 0) {
            issue_range.template operator()<0, LPW>(w);
          } else if constexpr (!MX) {
            // bf16, one MFMA step (a quarter of the window's K) at a time: the weights of step st + 1
            // are converted to bf16 and its A operands read ahead of the MFMAs of step st, so after the
            // window's barrier the matrix core waits for one step's conversion rather than the
            // whole window's
            float scl[PPW][4];
            #pragma unroll
            for (int pp = 0; pp < PPW; ++pp)
              #pragma unroll
              for (int ct = 0; ct < 4; ++ct) scl[pp][ct] = e8m0_f32((bsc[pp] >> (8 * ct)) & 0xFFu);
            u32x4 ac[N], an[N];
            bf16x8 bc[PPW][4], bn[PPW][4];
            auto read_slice = [&](const int st, u32x4 (&a)[N], bf16x8 (&b)[PPW][4]) __attribute__((always_inline)) {
              #pragma unroll
              for (int j = 0; j < N; ++j)
                a[j] = *(const u32x4*)(prow + j * NPH * 16 * AROW + 16 * ((4 * g + st) ^ (i16 & SWZ)));
              #pragma unroll
              for (int pp = 0; pp < PPW; ++pp)
                #pragma unroll
                for (int ct = 0; ct < 4; ++ct) b[pp][ct] = fp4_operand(bw[pp][ct][st], scl[pp][ct]);
            };  // step st: the A operands of the wave's tiles and the weights of its panels
            read_slice(0, ac, bc);
            [&]<int... SI>(std::integer_sequence<int, SI...>) {
              ([&] {
                constexpr int st = SI;
                if constexpr (st + 1 < 4) read_slice(st + 1, an, bn);
                #pragma unroll
                for (int j = 0; j < N; ++j)
                  #pragma unroll
                  for (int pp = 0; pp < PPW; ++pp)
                    #pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                      acc[j][pp][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ac[j]), bc[pp][ct],
                                                                                acc[j][pp][ct], 0, 0, 0);
                issue_range.template operator()<st * LPW / 4, (st + 1) * LPW / 4>(w);
                if constexpr (st + 1 < 4) {
                  #pragma unroll
                  for (int j = 0; j < N; ++j) ac[j] = an[j];
                  #pragma unroll
                  for (int pp = 0; pp < PPW; ++pp)
                    #pragma unroll
                    for (int ct = 0; ct < 4; ++ct) bc[pp][ct] = bn[pp][ct];
                }
              }(), ...);
            }(std::make_integer_sequence<int, 4>{});
          } else {
            // MXFP8: one scaled MFMA per tile and column tile covers the window; the next tile's
            // operands are read ahead
            i32x8 cur;
            int csc;
            load_tile(0, cur, csc);
            [&]<int... JI>(std::integer_sequence<int, JI...>) {
              ([&] {
                constexpr int j = JI;
                i32x8 nxt;
                int nsc = 0;
                if constexpr (j + 1 < N) load_tile(j + 1, nxt, nsc);
                #pragma unroll
                for (int pp = 0; pp < PPW; ++pp)
                  #pragma unroll
                  for (int ct = 0; ct < 4; ++ct) {
                    const i32x8 bop = {(int)bw[pp][ct][0], (int)bw[pp][ct][1], (int)bw[pp][ct][2], (int)bw[pp][ct][3],
                                       0, 0, 0, 0};
                    acc[j][pp][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        cur, bop, acc[j][pp][ct], 0, 4, 0, csc, 0, (int)(bsc[pp] >> (8 * ct)));
                  }
                issue_range.template operator()<j * LPW / N, (j + 1) * LPW / N>(w);
                if constexpr (j + 1 < N) {
                  cur = nxt;
                  csc = nsc;
                }
              }(), ...);
            }(std::make_integer_sequence<int, N>{});
          }
        }
      };
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((nw == I ? (run.template operator()<I>(), 0) : 0), ...);
      }(std::make_integer_sequence<int, MTW + 1>{});
      wait_vmcnt<0>();
      __syncthreads();  // rings idle
      // The next unit's prologue DMAs go out before this unit's epilogue (into A stages 0 .. DA - 1 and
      // the B stages; the epilogue stages in A stage NA - 1), so the memory path keeps working while
      // the epilogue computes; the full drain below holds whatever order loads and stores finish in.
      const int e_mb = mb, e_r1 = r1, e_panel0 = panel0, e_npan = npan, e_grp = grp;
      have = next_unit();
      if (have) prologue();
      finish(e_mb, e_r1, e_panel0, e_npan, e_grp);
      wait_vmcnt<0>();
      __syncthreads();  // staging and rings are reused by the next unit
  }
}


// Row-tiled grouped GEMM for MXFP8 activations (prefill gate/up and down): MXFP4 weights against
// E4M3 activation rows on the scaled MFMA, with the weights kept out of LDS.
// Block: 8 waves (2 per SIMD) on one expert's chunk of up to 192 rows and 4 consecutive panels; wave
// (pg, h) computes panel panel0 + pg on row tiles h, h + 2, ... (6 row tiles x 4 column tiles of 16).
// Per 128-K window:
//   - the two waves of a panel split its panel-window: wave h loads weight row-tiles 2h and 2h + 1 (and
//     the scale word) straight into a register ring DB windows ahead with the non-temporal policy (the
//     weights stream from HBM once; each lane's 16 bytes are already its MFMA operand), writes its two
//     row-tiles to an LDS stage at the end of the window before they are used and reads the partner's
//     two from there; so each weight byte passes the CU's load path once (that path moves about 55-64
//     bytes a clock per CU, LDS reads about three times as much);
//   - the chunk's activation rows (E4M3 codes and E8M0 scales, mostly L2 hits: the expert's other
//     panel blocks read the same rows) are loaded into registers DA windows ahead, each wave 24 rows
//     (three 16-byte pieces a lane, and one scale word a lane: real for waves 0..2, an out-of-range
//     load for the others), and written to one of two LDS stages the window before they are used
//     (16-byte chunk c of row r at position c ^ (r & 7), so the operand reads are conflict-free); all
//     eight waves read the operands of their tiles from it.
// Every load is compiler-visible and none sits under a branch inside a window, so the compiler's waits
// cover the loads a use depends on; one LDS wait and one barrier per window order the stages. Units (expert, chunk, panel block) come
// from the XCD's work-item list as in tiled_gemm_kernel; the next unit's first loads are issued before
// the current unit's epilogue.
// EPI 0: fp32 out. EPI 1: GLU panels, SiLU(gate) * up MX-encoded (E4M3, E8M0 per 32 units), staged in
// LDS and written as 16-byte row segments.

template <int NWAVE, int MT, int DA, int DB, int EPI, int TAG>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(NWAVE / 4, NWAVE / 4)))
void tiled_f8_kernel(GemmArgs args) {
  constexpr int ROWS = 16 * MT, NPG = 4, NPH = NWAVE / NPG, MTW = MT / NPH;
  constexpr int AROW = 128, A_SC = ROWS * AROW, A_STAGE = A_SC + ROWS * 4;
  constexpr int NB = DB + 1;
  static_assert(NPH == 2, "the two waves of a panel share its weight windows");
  constexpr int APL = ROWS * AROW / (16 * 64 * NWAVE);  // 16-byte activation pieces per lane and window
  constexpr int SCW = ROWS / 64;                         // waves that load a scale word per lane
  constexpr int U = NB % 2 == 0 ? NB : 2 * NB;           // windows per unrolled step (stage, set, slot cycle)
  static_assert(APL * 16 * 64 * NWAVE == ROWS * AROW && ROWS % 64 == 0 && U % DA == 0 && (DA == 1 || DA == 2),
                "shape");
  static_assert(ROWS * 132 <= A_STAGE, "epilogue staging fits one stage");
  static_assert(EPI == 0 || EPI == 1, "epilogue");
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][NPG][4096];  // weight codes, row-tile rt at 1024 rt
  __shared__ __attribute__((aligned(16))) uint8_t lds_sink[256];          // scale words of waves without scales

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pg = wv % NPG, h = wv / NPG;
  // column tile (weight row-tile) of the wave's MFMA slot q: its own two row-tiles first, then the
  // partner's (uniform over the wave)
  auto ctq = [&](int q) __attribute__((always_inline)) { return q < 2 ? 2 * h + q : 2 * (1 - h) + q - 2; };
  const int g = lane >> 4, i16 = lane & 15;
  const rsrc_t ar = make_rsrc(args.A, args.a_bytes);
  const rsrc_t asr = make_rsrc(args.A_scales, args.as_bytes);
  const int nwin = args.wwin;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const bool listed = args.items != nullptr;
  const int nblk = (args.P + 3) / 4;
  int it = 0, it_end = 0, it_step = 1;
  int cgrp = 0, cpanel0 = 0, cmb = 0, cr1 = 0;
  if (listed) {
    it = args.items[xcd] + slot;
    it_end = args.items[xcd + 1];
    it_step = (int)gridDim.x / 8;
  } else {
    const bool spread = args.n_groups < 8;
    cgrp = spread ? (int)blockIdx.x / nblk : xcd + 8 * (slot / nblk);
    cpanel0 = 4 * (spread ? (int)blockIdx.x % nblk : slot % nblk);
    if (cgrp >= args.n_groups) return;
    cmb = args.offsets[cgrp];
    cr1 = args.offsets[cgrp + 1];
    if (cmb >= cr1) return;
    if (cr1 - cmb < args.row_split || (args.row_cap > 0 && cr1 - cmb >= args.row_cap)) return;
  }
  // the unit in hand and the per-lane sources of its loads
  int grp = 0, panel0 = 0, mb = 0, r1 = 0, npan = 0;
  rsrc_t wr = make_rsrc(nullptr, 0);
  int aoff[APL], soff = -1;
  auto next_unit = [&]() __attribute__((always_inline)) -> bool {
    if (listed) {
      if (it >= it_end) return false;
      const u32 item = (u32)args.items[kItemHeader + it];
      it += it_step;
      grp = (int)(item & 0xFFFu);
      panel0 = 4 * (int)(item >> 24);
      mb = args.offsets[grp] + ROWS * (int)((item >> 12) & 0xFFFu);
      r1 = min(mb + ROWS, args.offsets[grp + 1]);
    } else {
      if (cmb >= cr1) return false;
      grp = cgrp;
      panel0 = cpanel0;
      mb = cmb;
      r1 = cr1;
      cmb += ROWS;
    }
    grp = __builtin_amdgcn_readfirstlane(grp);
    panel0 = __builtin_amdgcn_readfirstlane(panel0);
    mb = __builtin_amdgcn_readfirstlane(mb);
    r1 = __builtin_amdgcn_readfirstlane(r1);
    npan = min(4, args.P - panel0);
    // this wave's panel (zeros when the panel block is short)
    wr = make_rsrc(args.W + (int64_t)grp * args.w_group_stride + (int64_t)(panel0 + pg) * nwin * kPanelWinBytes,
                   pg < npan ? (int64_t)nwin * kPanelWinBytes : 0);
    // activation piece j of this lane: chunk row 24 wv + 8 j + lane / 8, LDS position lane % 8 holding the
    // row's 16-byte chunk (lane % 8) ^ (row & 7); rows past the chunk read zeros
#pragma unroll
    for (int j = 0; j < APL; ++j) {
      const int r = (ROWS / NWAVE) * wv + 8 * j + lane / 8;
      const int c = (lane % 8) ^ (r & 7);
      aoff[j] = mb + r < r1 ? (args.rowmap ? args.rowmap[mb + r] : mb + r) * (int)args.lda + 16 * c : -1;
    }
    if (wv < SCW) {
      const int r = 64 * wv + lane;
      soff = mb + r < r1 ? (args.rowmap ? args.rowmap[mb + r] : mb + r) * (int)args.ldas : -1;
    }
    return true;
  };

  struct AWinR {  // one window's activation pieces of this lane
    u32x4 c[APL];
    u32 sc;
  };
  struct BHalfR {  // one window of this wave's half of its panel: row-tiles 2h, 2h + 1 and the scales
    u32x4 c[2];
    u32 sc;
  };
  AWinR ast[DA];
  BHalfR bring[NB];
  // The window index passes through an empty asm statement: the offsets are then formed where the loads
  // are issued instead of being precomputed for every unrolled window (which would hold them in VGPRs).
  auto load_a = [&](AWinR& a, int w) __attribute__((always_inline)) {
    asm volatile("" : "+s"(w));
    const bool in = w < nwin;
#pragma unroll
    for (int j = 0; j < APL; ++j)
      a.c[j] = __builtin_amdgcn_raw_buffer_load_b128(ar, in && aoff[j] >= 0 ? aoff[j] + AROW * w : kOOB, 0, 0);
    // every wave issues the scale load (zeros past the chunk's scale rows), so the count of loads per
    // window is the same on every path and the compiler's load waits stay exact
    a.sc = __builtin_amdgcn_raw_buffer_load_b32(asr, in && soff >= 0 ? soff + 4 * w : kOOB, 0, 0);
  };
  auto store_a = [&](const AWinR& a, int stage) __attribute__((always_inline)) {
    uint8_t* base = &lds_a[stage][0];
#pragma unroll
    for (int j = 0; j < APL; ++j) *(u32x4*)(base + 1024 * (APL * wv + j) + 16 * lane) = a.c[j];
    *(u32*)((wv < SCW ? base + A_SC + 256 * wv : &lds_sink[0]) + 4 * lane) = a.sc;
  };
  auto load_b = [&](BHalfR& b, int w) __attribute__((always_inline)) {
    asm volatile("" : "+s"(w));
    const int off = w < nwin ? w * kPanelWinBytes : kOOB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      b.c[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, off + (2 * h + i) * 1024 + lane * 16, 0, kNT);
    b.sc = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 4096 + lane * 4, 0, kNT);
  };
  auto store_b = [&](const BHalfR& b, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4*)(&lds_b[stage][pg][(2 * h + i) * 1024 + 16 * lane]) = b.c[i];
  };
  // first loads of a unit: A(0), A(1) into the staging sets, B(0 .. DB - 1) into the ring
  auto prologue_loads = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < DA; ++n) load_a(ast[n], n);
#pragma unroll
    for (int n = 0; n < DB; ++n) load_b(bring[n], n);
  };
  // A(0) and this wave's half of B(0) to stage 0, then A(DA) into the set it came from (one set: A(1)
  // once A(0) is written)
  auto prologue_store = [&]() __attribute__((always_inline)) {
    store_a(ast[0], 0);
    store_b(bring[0], 0);
    load_a(ast[0], DA);
  };

  f32x4 acc[MTW][4];
  bool have = next_unit();
  if (have) {
    prologue_loads();
    prologue_store();
  }
  while (have) {
    const int nt = min(MT, (r1 - mb + 15) / 16);
    const int nw = nt > h ? (nt - h + NPH - 1) / NPH : 0;  // this wave's row tiles holding rows
#pragma unroll
    for (int j = 0; j < MTW; ++j)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The window loop, U windows unrolled. No load or stage write sits under a branch inside a window (at
    // the last window the stage writes carry the zeros of windows past K into stages nobody reads), so
    // the compiler's load waits cover exactly what each use needs rather than the loads just issued.
    auto run = [&]<int N>() __attribute__((always_inline)) {
      for (int w0 = 0; w0 < nwin; w0 += U) {
        [&]<int... UI>(std::integer_sequence<int, UI...>) __attribute__((always_inline)) {
          ([&]() __attribute__((always_inline)) {
            constexpr int u = UI;
            const int w = w0 + u;
            if (w < nwin) {  // uniform
              lds_barrier();  // A(w), B(w) in their stages for every wave; every wave done with window w - 1
              store_a(ast[(u + 1) % DA], (u + 1) & 1);
              load_a(ast[(u + 1) % DA], w + 1 + DA);
              load_b(bring[(u + DB) % NB], w + DB);
              if constexpr (N > 0) {
                const BHalfR& bw = bring[u % NB];
                // the partner's two row-tiles of B(w)
                const uint8_t* sbp = &lds_b[u & 1][pg][(2 - 2 * h) * 1024 + 16 * lane];
                const u32x4 bo[2] = {*(const u32x4*)sbp, *(const u32x4*)(sbp + 1024)};
                int bsq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) bsq[q] = (int)(bw.sc >> (8 * ctq(q)));
                const uint8_t* sa = lds_a[u & 1];
                const uint8_t* prow = sa + i16 * AROW + h * 16 * AROW;
                const uint8_t* psc = sa + A_SC + i16 * 4 + g + h * 64;
                auto tile = [&](int j, i32x8& op, int& sc) __attribute__((always_inline)) {
                  const uint8_t* pr = prow + j * NPH * 16 * AROW;
                  const u32x4 lo = *(const u32x4*)(pr + 16 * (g ^ (i16 & 7)));
                  const u32x4 hi = *(const u32x4*)(pr + 16 * ((4 + g) ^ (i16 & 7)));
                  sc = psc[j * NPH * 64];
                  op = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                };
                i32x8 cur;
                int csc;
                tile(0, cur, csc);
                [&]<int... JI>(std::integer_sequence<int, JI...>) __attribute__((always_inline)) {
                  ([&]() __attribute__((always_inline)) {
                    constexpr int j = JI;
                    i32x8 nxt;
                    int nsc = 0;
                    if constexpr (j + 1 < N) tile(j + 1, nxt, nsc);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                      const u32x4 bq = q < 2 ? bw.c[q] : bo[q - 2];
                      const i32x8 bop = {(int)bq[0], (int)bq[1], (int)bq[2], (int)bq[3], 0, 0, 0, 0};
                      acc[j][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur, bop, acc[j][q], 0, 4, 0, csc, 0,
                                                                                   bsq[q]);
                    }
                    if constexpr (j + 1 < N) {
                      cur = nxt;
                      csc = nsc;
                    }
                  }(), ...);
                }(std::make_integer_sequence<int, N>{});
              }
              // this wave's half of B(w + 1) to its stage after the window's MFMAs: its loads, issued two
              // windows before it is used, have had the most time to land
              store_b(bring[(u + 1) % NB], (u + 1) & 1);
            }
          }(), ...);
        }(std::make_integer_sequence<int, U>{});
      }
    };
    [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
      ((nw == I ? (run.template operator()<I>(), 0) : 0), ...);
    }(std::make_integer_sequence<int, MTW + 1>{});

    // Every wave done with the stages; the next unit's first loads go out before this unit's epilogue
    // (which stages in LDS) and its first LDS write after it.
    lds_barrier();
    const int e_mb = mb, e_r1 = r1, e_panel0 = panel0, e_npan = npan, e_grp = grp;
    have = next_unit();
    // the GLU epilogue's arithmetic covers the next unit's first loads; the fp32 one is only stores
    if (EPI == 1 && have) prologue_loads();
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));  // lane indices re-derived so no address arithmetic is hoisted
      const int eg = ln >> 4, ej = ln & 15;
      const EpiSeg& sg = args.seg[0];
      const int nrow = min(ROWS, e_r1 - e_mb);
      // LoRA deltas (the row-tiled launches need whole 64-column panels, so every column of a panel
      // below npan is a real one)
      if (args.lora_t) {
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
          const int row0 = e_mb + 16 * (h + NPH * j) + 4 * eg;
          if (pg < e_npan && row0 < e_r1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int ct = ctq(q);
              const int col = EPI == 1 ? 32 * (e_panel0 + pg) + 16 * (ct >> 1) + ej : 64 * (e_panel0 + pg) + 16 * ct + ej;
              const int q0 = EPI == 1 && (ct & 1) ? args.lora_rank : 0;
              lora_add(args, acc[j][q], e_grp, row0, e_r1, col, q0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (EPI == 1) {
        // codes staged as [ROWS][128 bytes] (32 units per panel), scales as [ROWS][4]
        uint8_t* stg = &lds_a[0][0];
        uint8_t* stg_sc = stg + ROWS * 128;
        // slots 0, 1 hold gate and up of units 32 pg + 16 h + ej (staging column ca), slots 2, 3 those of
        // units 32 pg + 16 (1 - h) + ej (column cb); the MX block is the 32 units of the panel either way
        const int ca = 32 * pg + 16 * h + ej, cb = 32 * pg + 16 * (1 - h) + ej;
        // TAP: also the fp32 SwiGLU values (a test tap); a separate copy of the loop, so the untapped one
        // carries none of its stores or branches
        auto glu = [&]<bool TAP>() __attribute__((always_inline)) {
          const rsrc_t prr = make_rsrc(TAP ? sg.pre + (int64_t)e_mb * sg.ldpre : nullptr, TAP ? (int64_t)nrow * sg.ldpre * 4 : 0);
#pragma unroll
          for (int j = 0; j < MTW; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float va = silu(acc[j][0][r]) * acc[j][1][r];
              const float vb = silu(acc[j][2][r]) * acc[j][3][r];
              const int lr = 16 * (h + NPH * j) + 4 * eg + r;
              if constexpr (TAP) {
                const int o = lr * (int)sg.ldpre + sg.col0 + 32 * e_panel0;
                const bool ok = lr < nrow && pg < e_npan;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(va), prr, ok ? 4 * (o + ca) : kOOB, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vb), prr, ok ? 4 * (o + cb) : kOOB, 0, 0);
              }
              u32 c0, c1, sb;
              mxfp8_block(va, vb, c0, c1, sb);
              stg[lr * 128 + ca] = (uint8_t)c0;
              stg[lr * 128 + cb] = (uint8_t)c1;
              if (ej == 0) stg_sc[lr * 4 + pg] = (uint8_t)sb;  // the 16 lanes of the block agree
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        if (sg.pre)
          glu.template operator()<true>();
        else
          glu.template operator()<false>();
        lds_barrier();
        const int t = threadIdx.x;
        uint8_t* out = (uint8_t*)sg.out + sg.col0 + 32 * e_panel0;
#pragma unroll
        for (int q = 0; q < ROWS / (8 * NWAVE); ++q) {
          const int lr = 8 * NWAVE * q + t / 8, piece = t % 8;
          if (lr < nrow && piece < 2 * e_npan)
            *(u32x4*)(out + (int64_t)(e_mb + lr) * sg.ldo + 16 * piece) = *(const u32x4*)(stg + lr * 128 + 16 * piece);
        }
        for (int lr = t; lr < nrow; lr += 64 * NWAVE) {
          uint8_t* os = sg.out_scales + (int64_t)(e_mb + lr) * sg.ldos + sg.col0 / 32 + e_panel0;
          if (e_npan == 4)
            *(u32*)os = *(const u32*)(stg_sc + 4 * lr);
          else
            for (int p = 0; p < e_npan; ++p) os[p] = stg_sc[4 * lr + p];
        }
        lds_barrier();  // staging read by every wave before the next unit's first LDS write
      } else {
        const rsrc_t orr = make_rsrc((float*)sg.out + (int64_t)e_mb * sg.ldo + sg.col0, (int64_t)nrow * sg.ldo * 4);
        const int ldo = (int)sg.ldo;
#pragma unroll
        for (int j = 0; j < MTW; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lr = 16 * (h + NPH * j) + 4 * eg + r;
            const int base = 4 * (lr * ldo + 64 * (e_panel0 + pg) + ej);
            const bool rok = lr < nrow && pg < e_npan;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int ct = ctq(q);
              const bool ok = rok && 64 * (e_panel0 + pg) + 16 * ct + ej < sg.ncols;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][q][r]), orr, ok ? base + 64 * ct : kOOB, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (EPI == 0 && have) prologue_loads();
    if (have) prologue_store();
  }
}

// Skinny dense GEMM (at most 64 rows, e.g. a decode batch against x's or the output's weights).
// With few rows the weights are the whole stream and the activation window (64 rows x 128 K) is
// needed by every panel; fetched per panel it would cost several times the weights. A block of 8
// waves takes one panel block (4 panels); wave (p, kh) computes panel p over all row tiles for
// half of every K window (MFMA steps 2 kh, 2 kh + 1), so each weight is converted to a bf16
// operand once and two waves share each SIMD (one wave alone issues the bf16 MFMA at about half
// its rate). Each activation window goes to LDS once (LDS-DMA, 16-byte chunks XOR-swizzled by
// row) and is read by all eight waves; each wave streams its half panel-windows straight into a
// register ring (non-temporal loads). Both rings run DA windows ahead: loads complete in order, so
// waiting for an activation window also waits for every weight load issued before it.
// Split-K across blocks: the nblk x nwin panel-block windows, in that order, are dealt to the
// grid as equal contiguous ranges (never longer than a panel), so every CU streams the same share
// of weights whatever the panel count. A range covers at most two panel blocks; its loads run on
// across the boundary, and the sums of each segment (the two K halves added through LDS) are
// written as a partial tile to workspace slot 2 * block + segment (fp32, MFMA order: [4 row
// tiles][4 panels][4 column tiles][64 lanes] x 4). skinny_reduce_kernel then adds, for each panel,
// the partials of the blocks that cover it in block order (deterministic) and applies the panel's
// segment epilogue.
constexpr int kSkinnyBlocks = 256;  // one block per CU
constexpr int kSkinnyRows = 64;
constexpr int64_t kSkinnySlotBytes = 4 * 4 * 4 * 64 * 16;

template <int DA, int NB, int TAG>
__global__ __launch_bounds__(512) void skinny_gemm_kernel(GemmArgs args) {
  constexpr int NA = DA + 1, DB = NB - 1;
  constexpr int AROW = 256, CPR = 16, RPD = 4;  // bf16 row window: 256 bytes; 4 rows per 1 KB DMA
  constexpr int A_STAGE = kSkinnyRows * AROW;
  constexpr int APW = kSkinnyRows / RPD / 8;    // 2 activation DMAs per wave and step
  constexpr int BPW = 5;                        // the wave's half panel-window: four 8-byte and one 4-byte load
  constexpr int LPW = APW + BPW;
  // At step i the later of A(i) and B(i) must have landed (loads complete in order). DB > DA: A(i)
  // is the later one, followed by its step's weight loads and DA - 1 full steps; DB == DA: B(i)
  // comes last in its step, followed by DA - 1 full steps. Waiting for A(i) also waits for every
  // weight load issued before it, so the weights stay only DA - 1 windows ahead whatever DB is:
  // both rings are kept equally deep.
  constexpr int WAITN = (DB > DA ? BPW : 0) + (DA - 1) * LPW;
  static_assert(DB >= DA && DA >= 1 && WAITN < 64, "ring depths");
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[NA][A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_sink[8][256];
  __shared__ __attribute__((aligned(16))) f32x4 lds_x[4][4][4][64];  // K-half sums handed over at segment ends

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pw = wv & 3, kh = wv >> 2;  // panel of the block; K half of every window (MFMA steps 2 kh, 2 kh + 1)
  const int nwin = args.wwin, P = args.P;
  const int nblk = (P + 3) / 4;
  const int G = gridDim.x, b = blockIdx.x;
  const u32 U = (u32)(nblk * nwin);  // U (G + 1) < 2^31 (host check): 32-bit divisions
  const int u0 = (int)((u32)b * U / (u32)G), u1 = (int)((u32)(b + 1) * U / (u32)G);
  if (u0 >= u1) return;  // uniform; never taken with G <= U
  const int n = u1 - u0;
  const int q0 = (int)((u32)u0 / (u32)nwin), w0 = u0 - q0 * nwin;
  const int n0 = min(n, nwin - w0);  // windows of the first segment; the rest start panel block q0 + 1

  const rsrc_t wr = make_rsrc(args.W, (int64_t)P * nwin * kPanelWinBytes);
  const i32x4s ar = sgpr_rsrc(args.A, args.a_bytes);
  const int g = lane >> 4, i16 = lane & 15;
  const u32 lds_a0 = lds_addr(&lds_a[0][0]);
  const u32 lds_s = lds_addr(&lds_sink[wv][0]);

  // activation DMA jj of this wave covers rows RPD (wv APW + jj) .. + RPD - 1 (lane L: row + L / CPR,
  // position L % CPR holding chunk (L % CPR) ^ (row & 15): a tile's 16 rows read 16 bank groups); rows
  // past M read zeros
  int acode[APW], akel[APW];
#pragma unroll
  for (int jj = 0; jj < APW; ++jj) {
    const int r = RPD * (wv * APW + jj) + lane / CPR;
    const int c = (lane % CPR) ^ (r & 15);
    akel[jj] = 8 * c;
    acode[jj] = r < args.M ? r * (int)args.lda * 2 + 16 * c : -1;
  }
  const u32 a_w = lds_a0 + 1024 * (wv * APW);
  auto qw = [&](int j, int& q, int& w) {  // panel block and window of local step j
    q = j < n0 ? q0 : q0 + 1;
    w = j < n0 ? w0 + j : j - n0;
  };
  auto issue_a = [&](int i) {  // activation DMAs of step i + DA (placeholders in the prologue)
    const int ja = i + DA;
    if (ja < 0) {
#pragma unroll
      for (int jj = 0; jj < APW; ++jj) dma4<false>(ar, lds_s, kOOB);
    } else {
      int q, w;
      qw(ja, q, w);
      const u32 st = (u32)((ja % NA) * A_STAGE);
#pragma unroll
      for (int jj = 0; jj < APW; ++jj)
        dma16<false>(ar, a_w + st + 1024 * jj,
                     ja < n && acode[jj] >= 0 && kWinK * w + akel[jj] < args.K ? acode[jj] + AROW * w : kOOB);
    }
  };
  struct HalfWin {  // the wave's half of a panel-window: dwords 2 kh, 2 kh + 1 of every lane's 16 bytes
    u32x2 c[4];
    u32 sc;
  };
  auto load_b = [&](HalfWin& bb, int j) {  // step j (zeros past the range)
    int q, w;
    qw(j, q, w);
    const int panel = 4 * q + pw;
    const int off = j < n && panel < P ? (panel * nwin + w) * kPanelWinBytes : kOOB;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      bb.c[rt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wr, off + rt * 1024 + lane * 16 + 8 * kh, 0, kNT));
    bb.sc = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 4096 + lane * 4, 0, kNT);
  };

  const int nt = (min(args.M, kSkinnyRows) + 15) / 16;
  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const rsrc_t prr = make_rsrc(args.partial, args.partial_bytes);
  auto slot_off = [&](int slot, int t, int ct) { return (int)(slot * kSkinnySlotBytes) + (((t * 4 + pw) * 4 + ct) * 64 + lane) * 16; };
  // the accumulated segment out as a partial tile (upper K half handed to the lower through LDS);
  // accumulators cleared
  auto flush = [&](int slot) {
    if (kh == 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < nt) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) lds_x[pw][t][ct][lane] = acc[t][ct];
        }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nt) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[t][ct] + lds_x[pw][t][ct][lane]), prr,
                                                   slot_off(slot, t, ct), 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  HalfWin ring[NB];
  auto run = [&]<int NT>() {
    // prologue: steps -DB .. -1 in steady-state order (activation DMAs, then weight loads)
#pragma unroll
    for (int i = -DB; i < 0; ++i) {
      issue_a(i);
      load_b(ring[i + DB], i + DB);
    }
    // one step: wait for its activation window, the MFMAs (guarded: steps past the range only keep
    // the load pattern), then the loads of step i + DA / i + DB (unconditionally, so that the
    // compiler's own waits for the ring stay exact)
    auto compute = [&]<int u>(int i) {
      const HalfWin& cb = ring[u];
      const uint8_t* prow = lds_a[i % NA] + i16 * AROW;
      // row tile t, lane (i16, g), MFMA step st = 2 kh + s: K elements [32 g + 8 st, +8); the next
      // step's operands are read from LDS while this step's MFMAs run
      auto aload = [&](int t, int s) {
        return *(const u32x4*)(prow + t * 16 * AROW + 16 * ((4 * g + 2 * kh + s) ^ i16));
      };
      u32x4 a_cur[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) a_cur[t] = aload(t, 0);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 a_nxt[NT];
        if (st < 1) {
#pragma unroll
          for (int t = 0; t < NT; ++t) a_nxt[t] = aload(t, st + 1);
        }
        bf16x8 bv[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bv[ct] = fp4_operand(cb.c[ct][st], e8m0_f32((cb.sc >> (8 * ct)) & 0xFFu));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, a_cur[t]);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[ct], acc[t][ct], 0, 0, 0);
        }
        if (st < 1) {
#pragma unroll
          for (int t = 0; t < NT; ++t) a_cur[t] = a_nxt[t];
        }
      }
    };
    for (int i0 = 0; i0 < n; i0 += NB) {
      [&]<int... UI>(std::integer_sequence<int, UI...>) {
        ([&] {
          const int i = i0 + UI;
          wait_vmcnt<WAITN>();
          barrier_nowait();  // A(i) complete for every wave; the stage of step i - 1 is free
          if (i < n) compute.template operator()<UI>(i);
          // issued after the step's MFMAs, so that a full memory queue stalls the wave while the
          // matrix core works (the wave issues nothing else until the next wait)
          issue_a(i);
          load_b(ring[(UI + DB) % NB], i + DB);  // into the slot step i - 1 used
          if (i == n0 - 1 && n > n0) flush(2 * b);  // end of the first of two segments
        }(), ...);
      }(std::make_integer_sequence<int, NB>{});
    }
  };
  if (nt == 4)
    run.template operator()<4>();
  else if (nt == 3)
    run.template operator()<3>();
  else if (nt == 2)
    run.template operator()<2>();
  else
    run.template operator()<1>();
  flush(n > n0 ? 2 * b + 1 : 2 * b);
}

// Sum of the partial tiles of one (panel block, row tile) in block order, then the panel's segment
// epilogue. Block: 4 waves, wave p = panel p of panel block blockIdx.x, row tile blockIdx.y. The
// covering blocks are consecutive; their partials are loaded kSkinnyBatch at a time (all loads of
// a batch in flight, blocks past the last one read zeros) and added in block order.
constexpr int kSkinnyBatch = 8;
template <int TAG>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(GemmArgs args, int G) {
  const int lane = threadIdx.x & 63;
  const int p = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = blockIdx.x, t = blockIdx.y;
  const int panel = 4 * q + p;
  if (panel >= args.P) return;
  const int nwin = args.wwin;
  const u32 U = (u32)(((args.P + 3) / 4) * nwin);  // U (G + 1) < 2^31 (host check): 32-bit divisions
  const u32 ua = (u32)(q * nwin), ue = ua + (u32)nwin;
  // first and last block whose range meets [ua, ue): block(u) = the last block starting at or before
  // u (ranges start at floor(b U / G) and are never empty); only the first can start in the previous
  // panel block
  const int b_lo = (int)(((ua + 1) * (u32)G + U - 1) / U) - 1;
  const int b_hi = (int)((ue * (u32)G + U - 1) / U) - 1;
  const int seg_lo = (u32)b_lo * U / (u32)G < ua ? 1 : 0;
  const rsrc_t prr = make_rsrc(args.partial, args.partial_bytes);
  const int lo = ((t * 4 + p) * 4 * 64 + lane) * 16;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b0 = b_lo; b0 <= b_hi; b0 += kSkinnyBatch) {
    f32x4 v[kSkinnyBatch][4];
#pragma unroll
    for (int c = 0; c < kSkinnyBatch; ++c) {
      const int b = b0 + c;
      const int off = b <= b_hi ? (int)((2 * b + (b == b_lo ? seg_lo : 0)) * kSkinnySlotBytes) + lo : kOOB;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        v[c][ct] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prr, off == kOOB ? kOOB : off + ct * 1024, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < kSkinnyBatch; ++c)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] += v[c][ct];
  }
  epilogue(args, acc, panel, 16 * t, min(args.M, kSkinnyRows), lane, 0);
}

template <int KSPLIT, int AFMT, int NBUF, int MT, bool AHEAD, int TAG, int LR = 0, bool ASH = false>
static void launch_one(GemmArgs a, hipStream_t s) {
  constexpr int ppb = BlockShape<KSPLIT>::panels;
  const int pblocks = (int)ceil_div(a.P, ppb);
  dim3 grid;
  if (a.offsets) {
    grid = dim3((unsigned)pblocks, (unsigned)a.n_groups);
  } else {
    a.m_passes = (int)ceil_div(a.M, 16 * MT);
    grid = dim3((unsigned)(ceil_div(pblocks, 8) * 8 * a.m_passes));
  }
  hipLaunchKernelGGL((panel_gemm_kernel<KSPLIT, AFMT, NBUF, MT, AHEAD, LR, ASH, TAG>), grid,
                     dim3(64 * BlockShape<KSPLIT>::waves), 0, s, a);
}

// ---------------------------------------------------------------------------------------------
// Grouped GEMM for experts of a few tens of rows (between the decode weight stream and the row-tiled
// prefill tiles): the panel kernel's weight stream with up to MT 16-row tiles of A per pass.
// Block: 4 waves on one expert and 4 consecutive panels, wave p computing panel 4 pblock + p. Per 128-K
// window each wave takes its panel-window from a register ring (NBUF - 1 windows ahead, non-temporal;
// the lane's 16 bytes are its operand, converted once to bf16 and used by every tile) and a share of
// the expert's A rows (MT tiles; bf16: MT pieces of 16 bytes a lane; MXFP8: codes for waves 0 and 1,
// scale words for wave 2) in the same ring; the shares go to one of two LDS stages the window they are
// used (16-byte chunk c of tile row r at position c ^ r) and after one barrier every wave reads its
// operands from there. Only tiles holding rows issue MFMAs. Experts with rows in [row_split, row_cap)
// run here; the others return at once.
// ---------------------------------------------------------------------------------------------
template <int AFMT, int NBUF, int MT, int TAG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void panel_rows_kernel(GemmArgs args) {
  constexpr int TB = AFMT == A_BF16 ? 4096 : 2048;  // code bytes of one 16-row tile's window
  constexpr int ASTG = MT * (TB + (AFMT == A_BF16 ? 0 : 64));
  __shared__ __attribute__((aligned(16))) uint8_t ash[2][ASTG];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pblock = blockIdx.x, grp = blockIdx.y;
  const int r0 = args.offsets[grp], r1 = args.offsets[grp + 1];
  if (r1 - r0 < max(args.row_split, 1) || r1 - r0 >= args.row_cap || 4 * pblock >= args.P) return;  // uniform
  const int panel = 4 * pblock + wave;
  const bool panel_ok = panel < args.P;
  const int nwin = args.wwin;  // every wave runs every window (the barriers)
  const rsrc_t wr = make_rsrc(args.W + (int64_t)grp * args.w_group_stride + (int64_t)(panel_ok ? panel : 0) * nwin * kPanelWinBytes,
                              (int64_t)(panel_ok ? nwin : 0) * kPanelWinBytes);
  const rsrc_t ar = make_rsrc(args.A, args.a_bytes);
  const rsrc_t asr = make_rsrc(args.A_scales, args.A_scales ? args.as_bytes : 0);
  const int g = lane >> 4, i16 = lane & 15;
  // the lane's piece of each tile: bf16, chunk pc of row pr (all 256 lanes); MXFP8, chunk pc of row pr
  // for waves 0 and 1, the row's scale word for lanes 0..15 of wave 2
  const int pi = 64 * wave + lane;
  const int pr = AFMT == A_BF16 ? pi >> 4 : (wave < 2 ? pi >> 3 : (wave == 2 ? lane : 16));
  const int pc = AFMT == A_BF16 ? pi & 15 : pi & 7;
  const bool plane = pr < 16 && (AFMT == A_BF16 || wave < 2 || (wave == 2 && lane < 16));
  struct RB {
    WWin w;
    u32x4 p[MT];
  };
  for (int mb = r0; mb < r1; mb += 16 * MT) {
    const int nt = min(MT, (r1 - mb + 15) / 16);  // tiles holding rows (uniform)
    int parow[MT];
    bool pv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int row = mb + 16 * t + pr;
      pv[t] = plane && t < nt && row < r1;
      parow[t] = pv[t] ? (args.rowmap ? args.rowmap[row] : row) : 0;
    }
    f32x4 acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // pieces past K (a K tail inside the last window) read zeros; a wave whose share of a tile lies past
    // the expert's rows (its first row there, uniform) issues no load for it and stages zeros: the load
    // path is what bounds this kernel, and loads past a buffer's range still cost their issue
    const int share0 = AFMT == A_BF16 ? 4 * wave : (wave < 2 ? 8 * wave : (wave == 2 ? 0 : 16));
    auto load_rb = [&](RB& b, int wi) {
      load_w(b.w, wr, lane, wi);
      const bool in = wi < nwin;
      const int k0 = kWinK * wi;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (share0 >= 16 || mb + 16 * t + share0 >= r1) {  // uniform
          b.p[t] = u32x4{0u, 0u, 0u, 0u};
          continue;
        }
        if constexpr (AFMT == A_BF16) {
          const int off = in && pv[t] && k0 + 8 * pc < args.K ? (parow[t] * (int)args.lda + k0 + 8 * pc) * 2 : kOOB;
          b.p[t] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        } else if (wave < 2) {
          const int off = in && pv[t] && k0 + 16 * pc < args.K ? parow[t] * (int)args.lda + k0 + 16 * pc : kOOB;
          b.p[t] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        } else {
          u32 w = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kb = k0 / 32 + q;
            w |= (u32)__builtin_amdgcn_raw_buffer_load_b8(
                     asr, in && pv[t] && 32 * kb < args.K ? parow[t] * (int)args.ldas + kb : kOOB, 0, 0)
                 << (8 * q);
          }
          b.p[t] = u32x4{w, 0u, 0u, 0u};
        }
      }
    };
    auto store_pieces = [&](const RB& b, int stage) {
      uint8_t* st = &ash[stage][0];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < nt) {  // uniform
          if constexpr (AFMT == A_BF16) {
            *(u32x4*)(st + TB * t + 256 * pr + 16 * (pc ^ pr)) = b.p[t];
          } else if (wave < 2) {
            *(u32x4*)(st + TB * t + 128 * pr + 16 * (pc ^ (pr & 7))) = b.p[t];
          } else if (wave == 2 && lane < 16) {
            *(u32*)(st + MT * TB + 64 * t + 4 * pr) = b.p[t][0];
          }
        }
      }
    };
    auto compute = [&](const WWin& w, int stage) {
      const uint8_t* st = &ash[stage][0];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        bf16x8 wv[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) wv[rt] = fp4_operand(w.c[rt][s2], e8m0_f32((w.sc >> (8 * rt)) & 0xFFu));
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < nt) {  // uniform
            bf16x8 av;
            if constexpr (AFMT == A_BF16) {
              av = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + TB * t + 256 * i16 + 16 * ((4 * g + s2) ^ i16)));
            } else {
              // the step's 8 codes: K [32 g + 8 s2, +8) of the row, in chunk 2 g + s2 / 2
              const uint2 c8 = *(const uint2*)(st + TB * t + 128 * i16 + 16 * ((2 * g + s2 / 2) ^ (i16 & 7)) + 8 * (s2 & 1));
              const float sc = e8m0_f32(st[MT * TB + 64 * t + 4 * i16 + g]);
              u32x4 r;
              r[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, false));
              r[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, true));
              r[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, false));
              r[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, true));
              av = __builtin_bit_cast(bf16x8, r);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[t][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wv[rt], acc[t][rt], 0, 0, 0);
          }
        }
      }
    };
    RB buf[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load_rb(buf[i], i);
    for (int w0 = 0; w0 < nwin; w0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        load_rb(buf[(u + NBUF - 1) % NBUF], w0 + u + NBUF - 1);
        if (w0 + u < nwin) {  // uniform over the block
          // stage (w & 1) was last read in window w - 2, before every wave reached the barrier of w - 1
          store_pieces(buf[u], (w0 + u) & 1);
          lds_barrier();
          compute(buf[u].w, (w0 + u) & 1);
        }
      }
    }
    // every wave done with the stages before the next pass writes them
    lds_barrier();
    if (panel_ok) {
      for (int t = 0; t < nt; ++t) {
        f32x4 tile[4];
#pragma unroll
        for (int t2 = 0; t2 < MT; ++t2)
          if (t2 == t) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) tile[rt] = acc[t2][rt];
          }
        epilogue(args, tile, panel, mb + 16 * t, r1, lane, grp);
      }
    }
  }
}

// Experts of fewer than kMidRows rows (and at least the launch's row split) take panel_rows_kernel
// when the launch has no LoRA deltas; the row-tiled kernels keep the larger ones.
constexpr int kMidRows = 64;
template <int AFMT, int NBUF, int TAG>
static void launch_panel_rows(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((panel_rows_kernel<AFMT, NBUF, kMidRows / 16, TAG>), dim3((unsigned)ceil_div(a.P, 4), (unsigned)a.n_groups),
                     dim3(256), 0, s, a);
}
// Grouped panel launches: with LoRA deltas the instance whose rank class holds the rank (the deltas
// then go in by MFMA steps inside the kernel), otherwise the plain one.
template <int AFMT, int NBUF, int TAG>
static void launch_grouped_panel(const GemmArgs& a, hipStream_t s) {
  if (!a.lora_t && a.row_split > 1)  // some experts have several rows: the shared A tile
    launch_one<1, AFMT, NBUF, 1, true, TAG, 0, true>(a, s);  // several rows per expert: one A tile per block
  else if (!a.lora_t)
    launch_one<1, AFMT, NBUF, 1, true, TAG>(a, s);
  else if (a.lora_rank <= 16)
    launch_one<1, AFMT, NBUF, 1, true, TAG, 16>(a, s);
  else
    launch_one<1, AFMT, NBUF, 1, true, TAG, 32>(a, s);
}

// Grouped launches split their groups by row count (row_split): the row-tiled kernel takes the groups
// with many rows, the panel kernel the others. The row-tiled kernel needs whole K windows and 16-byte
// aligned activation rows; MXFP8: 4-byte aligned scale rows and, for the GLU output, 16-byte aligned
// output rows and scale rows 4-byte aligned at panel-block granularity. One epilogue segment of the
// given mode covering every panel; activation offsets in 32 bits.
static bool tiled_grouped_ok(const GemmArgs& a, int mode) {
  if (a.row_split <= 0 || !a.offsets || a.K % kWinK || a.a_bytes >= ((int64_t)1 << 31) - (1 << 24)) return false;
  if (a.nseg != 1 || a.seg[0].p0 != 0 || a.seg[0].p1 < a.P || a.seg[0].mode != mode) return false;
  const EpiSeg& sg = a.seg[0];
  if (a.a_fmt == A_BF16) return a.lda % 8 == 0;
  if (a.a_fmt != A_MXFP8 || a.lda % 16 || a.ldas % 4) return false;
  if (mode == EPI_SWIGLU_MXFP8)
    return sg.ldo % 16 == 0 && sg.col0 % 128 == 0 && sg.ldos % 4 == 0 && sg.ncols == 32 * a.P;
  return true;
}

// Work-item list of a grouped row-tiled launch (one block of 1024 threads): every expert whose row
// count is in [max(split, 1), cap) (cap 0: unbounded) contributes ceil(rows / ROWS) chunks x nblk panel
// blocks, listed in the order (expert, panel block, chunk); the list is cut into 8 equal contiguous
// runs, run x for XCD x: out[x] = start of run x, out[8] = the total. Equal runs keep the XCDs equally
// busy however the rows are spread over the experts (a few hot experts would otherwise load a few
// XCDs), and contiguous runs keep each expert on one or two XCDs: the chunks of a panel block are
// adjacent (its weights are read once per XCD) and an expert's panel blocks follow one another (its
// activation rows stay in that L2).
constexpr int kMinChunkRows = 64;
int64_t tile_items_bytes(int64_t max_rows, int n_groups, int nblk) {
  return 4 * (kItemHeader + (int64_t)nblk * (n_groups + max_rows / kMinChunkRows + 1));
}
bool tile_items_fit(int64_t max_rows_per_group, int n_groups, int nblk) {
  return n_groups >= 1 && n_groups <= 2048 && nblk >= 1 && nblk <= 256 && max_rows_per_group / kMinChunkRows < 4095;
}

__device__ __forceinline__ int tile_items_of(const int32_t* offsets, int E, int e, int split, int cap, int rows, int nblk,
                                             int& nch) {
  nch = 0;
  if (e >= E) return 0;
  const int c = offsets[e + 1] - offsets[e];
  if (c < max(split, 1) || (cap > 0 && c >= cap)) return 0;
  nch = (c + rows - 1) / rows;
  return nch * nblk;
}

__global__ __launch_bounds__(1024) void tile_items_kernel(const int32_t* __restrict__ offsets, int E, int split, int cap,
                                                          int rows, int nblk, int32_t* __restrict__ out) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int ept = (E + 1023) / 1024;  // experts per thread: t ept .. t ept + ept - 1
  int sum = 0, nch;
  for (int j = 0; j < ept; ++j) sum += tile_items_of(offsets, E, t * ept + j, split, cap, rows, nblk, nch);
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan over the threads
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int base = part[t] - sum;
  for (int j = 0; j < ept; ++j) {
    const int e = t * ept + j;
    const int n = tile_items_of(offsets, E, e, split, cap, rows, nblk, nch);
    for (int pb = 0; pb < nblk && n > 0; ++pb)
      for (int ck = 0; ck < nch; ++ck)
        out[kItemHeader + base + pb * nch + ck] = (int32_t)((u32)e | ((u32)ck << 12) | ((u32)pb << 24));
    base += n;
  }
  if (t < 9) out[t] = (int32_t)(((int64_t)t * part[1023]) / 8);
}

// A grouped row-tiled launch: with an item list, the list for this row band and chunk height, then
// a persistent grid of one block per CU; without, one block per (group, panel block).
constexpr int kItemGrid = 256;
template <int DA, int DB, int MT, int EPI, int TAG, int AF>
static void launch_grouped_tiled(const GemmArgs& a, hipStream_t s) {
  constexpr int WPS = 2, PPW = 1;
  const unsigned nblk = (unsigned)ceil_div(a.P, 4);
  unsigned grid = (unsigned)ceil_div(a.n_groups, 8) * 8 * nblk;
  if (a.items) {
    hipLaunchKernelGGL(tile_items_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.n_groups, a.row_split, a.row_cap,
                       16 * MT, (int)nblk, a.items);
    grid = kItemGrid;
  }
  hipLaunchKernelGGL((tiled_gemm_kernel<AF, false, DA, DB, MT, WPS, PPW, EPI, TAG>), dim3(grid), dim3(256 * WPS), 0,
                     s, a);
}

template <int EPI, int TAG>
static void launch_f8(const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI == 0) {
    // down (fp32 out): both operands through LDS-DMA; activation rows 3 windows ahead, weights 2
    launch_grouped_tiled<3, 2, 12, EPI, TAG, A_MXFP8>(a, s);
  } else {
    // gate/up: 192-row chunks on 8 waves, half panel-windows 2 windows ahead in registers, activation
    // rows 2 ahead
    constexpr int NW = 8, MT = 12, DB = 2, DA = 2;
    const unsigned nblk = (unsigned)ceil_div(a.P, 4);
    unsigned grid = (unsigned)ceil_div(a.n_groups, 8) * 8 * nblk;
    if (a.items) {
      hipLaunchKernelGGL(tile_items_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.n_groups, a.row_split, a.row_cap,
                         16 * MT, (int)nblk, a.items);
      grid = kItemGrid;
    }
    hipLaunchKernelGGL((tiled_f8_kernel<NW, MT, DA, DB, EPI, TAG>), dim3(grid), dim3(64 * NW), 0, s, a);
  }
}

// bf16 grouped, the weights converted to bf16 operands once per window. Experts below 64 rows: 64-row
// chunks with the weights 4 windows ahead (with few rows the kernel is a weight stream and the depth
// of the weight ring sets its rate); 64 rows or more: 128-row chunks, weights 2 windows ahead (the
// activation stages take the room). Two launches, each skipping the other's experts.
constexpr int kBf16SmallRows = 64;
template <int EPI, int TAG>
static void launch_bf16_grouped(const GemmArgs& a, hipStream_t s) {
  GemmArgs lo = a, hi = a;
  lo.row_cap = kBf16SmallRows;
  hi.row_split = std::max(a.row_split, kBf16SmallRows);
  hi.row_cap = 0;
  if (a.row_split < kBf16SmallRows) launch_grouped_tiled<3, 4, 4, EPI, TAG, A_BF16>(lo, s);
  launch_grouped_tiled<2, 2, 8, EPI, TAG, A_BF16>(hi, s);
}

// Dense bf16 launches (beyond the skinny kernel's rows) take the row-tiled kernel; rows must be 16-byte
// aligned. With 1024 rows or more: 128-row chunks (at least 8, one XCD each); fewer: 64-row chunks
// with the weights 4 windows ahead (few chunks: the kernel is mostly a weight stream).
constexpr int kDenseRows = 128;
static bool dense_tiled_ok(const GemmArgs& a) {
  return !a.offsets && a.a_fmt == A_BF16 && a.M > 0 && a.lda % 8 == 0 && a.K % 32 == 0 &&
         a.a_bytes < ((int64_t)1 << 31) - (1 << 24);
}

template <int TAG>
static void launch_dense_tiled(const GemmArgs& a, hipStream_t s) {
  constexpr int WPS = 2, PPW = 1;
  const unsigned nblk = (unsigned)ceil_div(a.P, 4);
  if (a.M >= 8 * kDenseRows) {
    // 128-row chunks, chunk first (chunk c on XCD c mod 8, its activation rows read from that L2)
    GemmArgs b = a;
    b.panel_major = 0;
    const unsigned g8 = (unsigned)ceil_div(ceil_div(a.M, kDenseRows), 8) * 8;
    hipLaunchKernelGGL((tiled_gemm_kernel<A_BF16, true, 2, 2, kDenseRows / 16, WPS, PPW, 2, TAG>), dim3(g8 * nblk),
                       dim3(256 * WPS), 0, s, b);
  } else {
    // 64-row chunks, panel-major: the grid covers every (panel block, chunk), XCD by XCD
    GemmArgs b = a;
    b.panel_major = 1;
    const unsigned nch = (unsigned)ceil_div(a.M, 64);
    hipLaunchKernelGGL((tiled_gemm_kernel<A_BF16, true, 3, 4, 4, WPS, PPW, 2, TAG>), dim3(ceil_div(nblk, 8) * 8 * nch),
                       dim3(256 * WPS), 0, s, b);
  }
}

// Dense bf16 launches of at most 64 rows take the split-K skinny kernel when the workspace for its
// partial sums is there and the panel blocks fit the block count (ranges no longer than a panel).
int64_t gemm_partial_bytes() { return 2 * kSkinnyBlocks * kSkinnySlotBytes; }
static bool skinny_ok(const GemmArgs& a) {
  return !a.offsets && a.a_fmt == A_BF16 && a.M <= kSkinnyRows && a.lda % 8 == 0 && a.K % 32 == 0 &&
         a.partial && a.partial_bytes >= gemm_partial_bytes() &&
         ceil_div(a.P, 4) <= kSkinnyBlocks && ceil_div(a.P, 4) * a.wwin * (kSkinnyBlocks + 1) < ((int64_t)1 << 31) &&
         a.a_bytes < (int64_t)1 << 30 && (int64_t)a.P * a.wwin * kPanelWinBytes < (int64_t)1 << 30;
}

template <int TAG>
static void launch_skinny(const GemmArgs& a, hipStream_t s) {
  constexpr int DA = 2, NB = 3;  // deeper rings measured no faster
  const int nblk = (int)ceil_div(a.P, 4);
  const int G = (int)std::min<int64_t>(kSkinnyBlocks, (int64_t)nblk * a.wwin);  // nblk <= G <= windows
  hipLaunchKernelGGL((skinny_gemm_kernel<DA, NB, TAG>), dim3(G), dim3(512), 0, s, a);
  hipLaunchKernelGGL((skinny_reduce_kernel<TAG>), dim3(nblk, (unsigned)ceil_div(a.M, 16)), dim3(256), 0, s, a, G);
}

hipError_t launch_panel_gemm(const GemmArgs& a, GemmStage stage, hipStream_t s) {
  if (a.P <= 0) return hipSuccess;
  if (a.offsets == nullptr && a.M <= 0) return hipSuccess;
  switch (stage) {
    case GEMM_X:
      if (skinny_ok(a))
        launch_skinny<GEMM_X>(a, s);
      else if (dense_tiled_ok(a))
        launch_dense_tiled<GEMM_X>(a, s);
      else
        launch_one<8, A_BF16, 3, 1, true, GEMM_X>(a, s);
      break;
    case GEMM_Y:
      if (skinny_ok(a))
        launch_skinny<GEMM_Y>(a, s);
      else if (dense_tiled_ok(a))
        launch_dense_tiled<GEMM_Y>(a, s);
      else
        launch_one<8, A_BF16, 3, 1, true, GEMM_Y>(a, s);
      break;
    case GEMM_GATEUP:
    case GEMM_DOWN: {
      const bool gu = stage == GEMM_GATEUP;
      const bool bf = a.a_fmt == A_BF16;
      const int mode = gu ? (bf ? EPI_SWIGLU_BF16 : EPI_SWIGLU_MXFP8) : EPI_F32;
      GemmArgs pa = a;  // the panel kernel's share
      if (tiled_grouped_ok(a, mode)) {
        // without LoRA deltas: experts of [row_split, kMidRows) rows on panel_rows_kernel, larger ones
        // on the row-tiled kernels
        // (not when the average group holds 2 kMidRows rows or more: groups below kMidRows are then rare
        // and a launch of one block per (panel block, group) that mostly returns at once costs more)
        const bool mid = !a.lora_t && (a.M <= 0 || a.M < (int64_t)2 * kMidRows * a.n_groups);
        GemmArgs ta = a;
        if (mid) {
          ta.row_split = std::max(a.row_split, kMidRows);
          GemmArgs ma = a;
          ma.row_cap = kMidRows;
          if (gu && bf)
            launch_panel_rows<A_BF16, 3, GEMM_GATEUP>(ma, s);
          else if (gu)
            launch_panel_rows<A_MXFP8, 3, GEMM_GATEUP>(ma, s);
          else if (bf)
            launch_panel_rows<A_BF16, 3, GEMM_DOWN>(ma, s);
          else
            launch_panel_rows<A_MXFP8, 3, GEMM_DOWN>(ma, s);
        }
        if (gu && bf)
          launch_bf16_grouped<2, GEMM_GATEUP>(ta, s);
        else if (gu)
          launch_f8<1, GEMM_GATEUP>(ta, s);
        else if (bf)
          launch_bf16_grouped<0, GEMM_DOWN>(ta, s);
        else
          launch_f8<0, GEMM_DOWN>(ta, s);
        if (a.row_split == 1) break;  // no group left for the panel kernel
      } else {
        pa.row_split = 0;
      }
      if (gu && bf)
        launch_grouped_panel<A_BF16, 4, GEMM_GATEUP>(pa, s);  // weights 3 windows ahead
      else if (gu)
        launch_grouped_panel<A_MXFP8, 3, GEMM_GATEUP>(pa, s);
      else if (bf)
        launch_grouped_panel<A_BF16, 4, GEMM_DOWN>(pa, s);  // weights 3 windows ahead
      else
        launch_grouped_panel<A_MXFP8, 3, GEMM_DOWN>(pa, s);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Router top-k (eq. 13): per token, the k largest keys s + b in descending order (equal keys:
// lower expert first), and p_j = s_j / sum of the selected s. One wave per token; lane l holds
// experts l, l + 64, ... Each (key, expert) pair is packed into one 64-bit integer that orders
// exactly like the rule (order-preserving key bits above, inverted expert id below), so a round
// is one wave max; only the lane that owned the winner rescans its entries.
// ---------------------------------------------------------------------------------------------
typedef unsigned long long u64;

__device__ __forceinline__ u64 topk_pack(float key, int e) {
  const u32 b = __float_as_uint(key);
  const u32 ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // monotone in key
  return ((u64)ord << 32) | (u64)(0xFFFFFFFFu - (u32)e);
}

// Maximum of a 64-bit value over the wave with DPP moves (quad swaps, half-row and row mirrors, then
// the row broadcasts 15 and 31 that carry each row's maximum into the next rows): lane 63 ends with
// the wave maximum, which readlane makes uniform. Lanes a move does not reach keep their value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ u64 dpp_max_step(u64 v) {
  const u32 lo = (u32)v, hi = (u32)(v >> 32);
  const u32 olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const u32 ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  const u64 o = ((u64)ohi << 32) | olo;
  return o > v ? o : v;
}
__device__ __forceinline__ u64 wave_max_u64(u64 v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror: every lane of a row holds the row maximum
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds the maximum
  const u32 lo = __builtin_amdgcn_readlane((u32)v, 63), hi = __builtin_amdgcn_readlane((u32)(v >> 32), 63);
  return ((u64)hi << 32) | lo;
}

template <int NPER>
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ scores, const float* __restrict__ bias,
                                                  int T, int E, int k, int32_t* __restrict__ idx,
                                                  float* __restrict__ p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  if (t >= T) return;  // uniform over the wave
  const float* srow = scores + (int64_t)t * E;
  float sv[NPER], bv[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {  // all loads in flight together (clamped index, no branch)
    const int e = min(lane + 64 * i, E - 1);
    sv[i] = srow[e];
    bv[i] = bias[e];
  }
  u64 key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    const float kk = sv[i] + bv[i];
    // entries past E rank below every real entry; a NaN key ranks with -inf
    key[i] = e < E ? topk_pack(kk == kk ? kk : -INFINITY, e) : 0ull;
  }
  u64 best = 0ull;
#pragma unroll
  for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
  int my_e = 0;
  for (int jj = 0; jj < k; ++jj) {
    const u64 w = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (u32)w);
    if (lane == jj) my_e = e;
    if ((e & 63) == lane) {  // the owner drops the winner and rescans
      best = 0ull;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        if (key[i] == w) key[i] = 0ull;
        best = key[i] > best ? key[i] : best;
      }
    }
  }
  const float my_s = lane < k ? srow[my_e] : 0.0f;
  float sum = my_s;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_e;
    p[(int64_t)t * k + lane] = my_s / sum;
  }
}

hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* idx, float* p,
                       hipStream_t s) {
  dim3 grid((unsigned)T);  // one wave per token
  const int nper = (int)ceil_div(E, 64);
  if (nper <= 1)
    hipLaunchKernelGGL((topk_kernel<1>), grid, dim3(64), 0, s, scores, bias, T, E, k, idx, p);
  else if (nper <= 4)
    hipLaunchKernelGGL((topk_kernel<4>), grid, dim3(64), 0, s, scores, bias, T, E, k, idx, p);
  else if (nper <= 14)
    hipLaunchKernelGGL((topk_kernel<14>), grid, dim3(64), 0, s, scores, bias, T, E, k, idx, p);
  else if (nper <= 32)
    hipLaunchKernelGGL((topk_kernel<32>), grid, dim3(64), 0, s, scores, bias, T, E, k, idx, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Dispatch tables: counts per expert, exclusive offsets, and the expert-contiguous row order
// (expert ascending, token ascending), without atomics whose order could change the result.
// One block of 1024 threads walks the tokens in chunks of 64: a 64-bit LDS mask per expert marks
// the chunk's tokens that chose it (ds_or), a token's rank inside its expert is the running
// base of the expert plus the popcount of the mask bits below it.
// ---------------------------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
constexpr int kMaxExperts = 2048;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int32_t base[kMaxExperts];
  __shared__ int32_t part[kRouteThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) base[e] = 0;
  for (int c0 = 0; c0 < T; c0 += 64) {
    const int ntok = min(64, T - c0);
    for (int e = tid; e < E; e += kRouteThreads) mask[e] = 0ull;
    __syncthreads();
    for (int q = tid; q < ntok * k; q += kRouteThreads) {
      const int e = min(max(idx[(int64_t)c0 * k + q], 0), E - 1);
      atomicOr(&mask[e], 1ull << (q / k));
    }
    __syncthreads();
    for (int q = tid; q < ntok * k; q += kRouteThreads) {
      const int e = min(max(idx[(int64_t)c0 * k + q], 0), E - 1);
      const int tl = q / k;
      const unsigned long long below = tl ? (mask[e] & ((1ull << tl) - 1ull)) : 0ull;
      inv[(int64_t)c0 * k + q] = base[e] + __popcll(below);  // rank inside the expert for now
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) base[e] += __popcll(mask[e]);
    __syncthreads();
  }
  // exclusive scan of base[0..E) -> offsets; each thread owns a contiguous run of experts
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int run = 0;
  for (int e = e0; e < e1; ++e) run += base[e];
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int acc = part[tid] - run;  // exclusive prefix of this thread's run
  for (int e = e0; e < e1; ++e) {
    counts[e] = base[e];
    offsets[e] = acc;
    const int c = base[e];
    base[e] = acc;  // reuse as the expert's first row
    acc += c;
  }
  if (tid == kRouteThreads - 1) offsets[E] = part[kRouteThreads - 1];
  __syncthreads();
  for (int q = tid; q < T * k; q += kRouteThreads) {
    const int e = min(max(idx[q], 0), E - 1);
    const int row = base[e] + inv[q];
    inv[q] = row;
    perm[row] = q / k;
  }
}

// The same tables for many tokens, in parallel over 64-token chunks (same result):
//   route_chunk:   per chunk, each entry's rank among the chunk's entries of its expert (64-bit
//                  LDS masks as above) and the chunk's count per expert;
//   route_scan:    per expert (one wave), the exclusive scan of its chunk counts over the chunks
//                  (the expert's rows before the chunk) and its total;
//   route_offsets: the exclusive scan of the totals over the experts;
//   route_scatter: row = offsets[e] + rows of e before the chunk + rank in the chunk.
constexpr int kRouteChunk = 64;

__global__ __launch_bounds__(256) void route_chunk_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                          int32_t* __restrict__ rank, int32_t* __restrict__ ccount) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int c = blockIdx.x, tid = threadIdx.x;
  const int t0 = c * kRouteChunk, ntok = min(kRouteChunk, T - t0);
  for (int e = tid; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  for (int q = tid; q < ntok * k; q += 256) {
    const int e = min(max(idx[(int64_t)t0 * k + q], 0), E - 1);
    atomicOr(&mask[e], 1ull << (q / k));
  }
  __syncthreads();
  for (int q = tid; q < ntok * k; q += 256) {
    const int e = min(max(idx[(int64_t)t0 * k + q], 0), E - 1);
    const int tl = q / k;
    rank[(int64_t)t0 * k + q] = tl ? __popcll(mask[e] & ((1ull << tl) - 1ull)) : 0;
  }
  for (int e = tid; e < E; e += 256) ccount[(int64_t)c * E + e] = __popcll(mask[e]);
}

__global__ __launch_bounds__(256) void route_scan_kernel(int nchunk, int E, int32_t* __restrict__ ccount,
                                                         int32_t* __restrict__ counts) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;  // uniform per wave
  int carry = 0;
  for (int c0 = 0; c0 < nchunk; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nchunk ? ccount[(int64_t)c * E + e] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (c < nchunk) ccount[(int64_t)c * E + e] = carry + incl - v;  // rows of e before chunk c
    carry += __shfl(incl, 63);
  }
  if (lane == 0) counts[e] = carry;
}

__global__ __launch_bounds__(kRouteThreads) void route_offsets_kernel(int E, const int32_t* __restrict__ counts,
                                                                      int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kRouteThreads];
  const int tid = threadIdx.x;
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int run = 0;
  for (int e = e0; e < e1; ++e) run += counts[e];
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int acc = part[tid] - run;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = acc;
    acc += counts[e];
  }
  if (tid == kRouteThreads - 1) offsets[E] = part[kRouteThreads - 1];
}

__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ cbase, int32_t* __restrict__ inv,
                                                            int32_t* __restrict__ perm) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)T * k) return;
  const int e = min(max(idx[q], 0), E - 1);
  const int t = (int)(q / k);
  const int row = offsets[e] + cbase[(int64_t)(t / kRouteChunk) * E + e] + inv[q];
  inv[q] = row;
  perm[row] = t;
}

int64_t route_scratch_bytes(int max_tokens, int E) {
  return (int64_t)ceil_div(max_tokens, kRouteChunk) * E * 4;
}

hipError_t launch_route(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv, int32_t* scratch, hipStream_t s) {
  if (E > kMaxExperts || k > kRouteChunk) return hipErrorInvalidValue;
  if (T <= 8 * kRouteChunk || scratch == nullptr) {
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, idx, T, E, k, counts, offsets, perm, inv);
    return hipGetLastError();
  }
  const int nchunk = (int)ceil_div(T, kRouteChunk);
  hipLaunchKernelGGL(route_chunk_kernel, dim3(nchunk), dim3(256), 0, s, idx, T, E, k, inv, scratch);
  hipLaunchKernelGGL(route_scan_kernel, dim3((unsigned)ceil_div(E, 4)), dim3(256), 0, s, nchunk, E, scratch, counts);
  hipLaunchKernelGGL(route_offsets_kernel, dim3(1), dim3(kRouteThreads), 0, s, E, (const int32_t*)counts, offsets);
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)ceil_div((int64_t)T * k, 256)), dim3(256), 0, s, idx, T, E,
                     k, (const int32_t*)offsets, (const int32_t*)scratch, inv, perm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine + RMSNorm (eq. 11): u_t = sum_j p_tj O[inv[t, j]] in selection order, then
// n_t = bf16(gamma * u_t / sqrt(mean(u_t^2) + eps)). One block per token.
// ---------------------------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
constexpr int kMaxWidth = 8192;
constexpr int kCombineChunks = kMaxWidth / (4 * kCombineThreads);  // float4 columns per thread, at most

// Four consecutive expert outputs, loaded non-temporal: each is read once (-11% at 8192 tokens).
__device__ __forceinline__ float4 load4_nt(const float* p) {
  return make_float4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1), __builtin_nontemporal_load(p + 2),
                     __builtin_nontemporal_load(p + 3));
}

// One block of 256 threads per token; thread tid holds columns 4 tid + 1024 i (i < 8) of u_t in
// registers. KC > 0: k fixed at compile time, so all of a chunk's row loads are in flight at once.
template <int KC>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ O,
                                                                  const int32_t* __restrict__ inv,
                                                                  const float* __restrict__ p, int k, int width,
                                                                  const float* __restrict__ gamma, float eps, int mode,
                                                                  u16* __restrict__ n_out, int64_t ldn,
                                                                  float* __restrict__ u_out) {
  __shared__ int32_t rows[64];
  __shared__ float pp[64];
  __shared__ float red[kCombineThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = inv[(int64_t)t * k + tid];
    pp[tid] = p[(int64_t)t * k + tid];
  }
  __syncthreads();
  float4 u[kCombineChunks];
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = 4 * tid + 4 * kCombineThreads * i;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < width) {
      if constexpr (KC > 0) {
        float4 o[KC];
#pragma unroll
        for (int jj = 0; jj < KC; ++jj) o[jj] = load4_nt(O + (int64_t)rows[jj] * width + c);
#pragma unroll
        for (int jj = 0; jj < KC; ++jj) {  // selection order, as the runtime-k loop
          const float w = pp[jj];
          a.x += w * o[jj].x;
          a.y += w * o[jj].y;
          a.z += w * o[jj].z;
          a.w += w * o[jj].w;
        }
      } else {
        for (int jj = 0; jj < k; ++jj) {
          const float4 o = load4_nt(O + (int64_t)rows[jj] * width + c);
          const float w = pp[jj];
          a.x += w * o.x;
          a.y += w * o.y;
          a.z += w * o.z;
          a.w += w * o.w;
        }
      }
      if (u_out) *(float4*)(u_out + (int64_t)t * width + c) = a;
      sq += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    u[i] = a;
  }
  if (mode != 0) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) tot += red[i];
  const float rs = 1.0f / sqrtf(tot / (float)width + eps);
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = 4 * tid + 4 * kCombineThreads * i;
    if (c < width) {
      const float4 gm = *(const float4*)(gamma + c);
      const u32 lo = bf16_rne(gm.x * u[i].x * rs) | (bf16_rne(gm.y * u[i].y * rs) << 16);
      const u32 hi = bf16_rne(gm.z * u[i].z * rs) | (bf16_rne(gm.w * u[i].w * rs) << 16);
      *(uint2*)(n_out + (int64_t)t * ldn + c) = make_uint2(lo, hi);
    }
  }
}

hipError_t launch_combine(const float* O, const int32_t* inv, const float* p, int T, int k, int width,
                          const float* gamma, float eps, int mode, uint16_t* n_out, int64_t ldn, float* u_out,
                          hipStream_t s) {
  if (width > kMaxWidth || k > 64 || width % 4 || (mode == 0 && ldn % 4)) return hipErrorInvalidValue;
  if (k == 16)
    hipLaunchKernelGGL(combine_kernel<16>, dim3(T), dim3(kCombineThreads), 0, s, O, inv, p, k, width, gamma, eps, mode,
                       n_out, ldn, u_out);
  else if (k == 8)
    hipLaunchKernelGGL(combine_kernel<8>, dim3(T), dim3(kCombineThreads), 0, s, O, inv, p, k, width, gamma, eps, mode,
                       n_out, ldn, u_out);
  else
    hipLaunchKernelGGL(combine_kernel<0>, dim3(T), dim3(kCombineThreads), 0, s, O, inv, p, k, width, gamma, eps, mode,
                       n_out, ldn, u_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Quantile Balancing ("Serving K3, 01 architecture", hot-expert paragraph; "Kimi K3: architectural
// innovations", "A router decision is also a scheduling decision"): expert allocation from
// router-score quantiles, read as b_e = -(the m-th largest score of expert e over a calibration
// batch), m = round(T k / E). One block per expert: the expert's T scores as order-preserving
// 32-bit keys in LDS, a bitonic sort into descending order (padding keys 0 sort last), then the
// key at rank m. The result is one of the scores, exactly.
// ---------------------------------------------------------------------------------------------
constexpr int kBalanceMaxTokens = 16384;

__device__ __forceinline__ u32 order_key(float f) {  // monotone in f (finite values)
  const u32 u = __float_as_uint(f);
  return u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float from_order_key(u32 k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__global__ __launch_bounds__(1024) void quantile_bias_kernel(const float* __restrict__ scores, int T, int E, int m,
                                                             float* __restrict__ bias) {
  __shared__ u32 keys[kBalanceMaxTokens];
  const int e = blockIdx.x, tid = threadIdx.x;
  int n = 1;
  while (n < T) n <<= 1;  // uniform; n <= kBalanceMaxTokens (host check)
  for (int i = tid; i < n; i += 1024) keys[i] = i < T ? order_key(scores[(int64_t)i * E + e]) : 0u;
  __syncthreads();
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n / 2; i += 1024) {
        const int lo = 2 * stride * (i / stride) + i % stride, hi = lo + stride;
        const bool desc = (lo & size) == 0;  // the merge directions that leave the whole array descending
        const u32 a = keys[lo], b = keys[hi];
        if ((a < b) == desc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) bias[e] = -from_order_key(keys[m - 1]);
}

hipError_t launch_quantile_bias(const float* scores, int T, int E, int m, float* bias, hipStream_t s) {
  if (T < 1 || T > kBalanceMaxTokens || E < 1 || m < 1 || m > T) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantile_bias_kernel, dim3((unsigned)E), dim3(1024), 0, s, scores, T, E, m, bias);
  return hipGetLastError();
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ in, u16* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (u16)bf16_rne(in[i]);
}

hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// BF16 LoRA deltas over the MXFP4 experts ("Serving K3, 01 architecture": fine-tuning ships bf16 LoRA
// deltas over the 4-bit base). The first factor t = act La^T of a grouped stage (rank columns per
// matrix); the second factor is added in the grouped GEMMs' epilogues (lora_add).
// One block of 4 waves per group: the group's rows in chunks of 64 (4 row tiles of 16); wave w takes
// K windows w, w + 4, ... of 128; in MFMA step st of a window, lane (i, g) holds K [128 w + 32 st + 8 g,
// +8) of row / column i (four bf16 MFMA 16x16x32 steps a window). The waves' sums are added in wave
// order through LDS (deterministic).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void lora_act_load(const LoraAArgs& a, rsrc_t ar, rsrc_t asr, int arow, bool ok, int w, int g,
                                              bf16x8 (&v)[4]) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int k0 = kWinK * w + 32 * st + 8 * g;  // the lane's 8 K elements of step st
    const bool in = ok && k0 < a.K;
    if (a.a_fmt == A_BF16) {
      v[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ar, in ? (arow * (int)a.lda + k0) * 2 : kOOB, 0, 0));
    } else {
      const int off = in ? arow * (int)a.lda + k0 : kOOB;
      const u32 d0 = __builtin_amdgcn_raw_buffer_load_b32(ar, off, 0, 0);
      const u32 d1 = __builtin_amdgcn_raw_buffer_load_b32(ar, off == kOOB ? kOOB : off + 4, 0, 0);
      const float sc = e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(asr, in ? arow * (int)a.ldas + k0 / 32 : kOOB, 0, 0));
      u32x4 r;
      r[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false));
      r[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true));
      r[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false));
      r[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true));
      v[st] = __builtin_bit_cast(bf16x8, r);
    }
  }
}

// One block of kLoraWaves waves per group; the K windows are dealt over the waves, each wave keeping the
// next window's weights (and its first row tile's activations) in flight while it computes the current
// one; the waves' partial sums are added in wave order through LDS (deterministic). NCT column tiles of 16.
constexpr int kLoraWaves = 4;
template <int NCT>
__global__ __launch_bounds__(64 * kLoraWaves) void lora_a_kernel(LoraAArgs a) {
  __shared__ f32x4 red[kLoraWaves][NCT][64];  // one row tile's partial sums of every wave
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = blockIdx.x;
  const int r0 = a.offsets[grp], r1 = a.offsets[grp + 1];
  if (r0 >= r1) return;  // uniform
  const int i16 = lane & 15, g = lane >> 4;
  const int nwin = (a.K + kWinK - 1) / kWinK;
  const rsrc_t ar = make_rsrc(a.A, a.a_bytes);
  const rsrc_t asr = make_rsrc(a.A_scales, a.A_scales ? a.as_bytes : 0);
  const rsrc_t lr = make_rsrc(a.La + (int64_t)grp * a.la_stride, (int64_t)a.N * a.K * 2);
  struct Win {
    bf16x8 b[NCT][4];
    bf16x8 a0[4];
  };
  for (int mb = r0; mb < r1; mb += 64) {
    const int nrt = min(4, (r1 - mb + 15) / 16);
    f32x4 acc[4][NCT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    int arow[4];
    bool aok[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = mb + 16 * rt + i16;
      aok[rt] = rt < nrt && row < r1;
      arow[rt] = aok[rt] ? (a.rowmap ? a.rowmap[row] : row) : 0;
    }
    // MFMA step st of window w: lane group g takes K elements [128 w + 32 st + 8 g, +8) on both operands,
    // so one load instruction reads 64 contiguous bytes of each of its 16 rows
    auto load_win = [&](Win& x, int w) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int n = 16 * ct + i16;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int k0 = kWinK * w + 32 * st + 8 * g;
          const int off = w < nwin && n < a.N && k0 < a.K ? (n * a.K + k0) * 2 : kOOB;
          x.b[ct][st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(lr, off, 0, 0));
        }
      }
      lora_act_load(a, ar, asr, arow[0], aok[0] && w < nwin, w, g, x.a0);
    };
    Win cur, nxt;
    load_win(cur, wv);
    for (int w = wv; w < nwin; w += kLoraWaves) {
      load_win(nxt, w + kLoraWaves);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt < nrt) {  // uniform
          bf16x8 av[4];
          if (rt == 0) {
#pragma unroll
            for (int st = 0; st < 4; ++st) av[st] = cur.a0[st];
          } else {
            lora_act_load(a, ar, asr, arow[rt], aok[rt], w, g, av);
          }
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
              acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st], cur.b[ct][st], acc[rt][ct], 0, 0, 0);
        }
      }
      cur = nxt;
    }
    // the waves' partial sums, one row tile at a time, added in wave order (deterministic)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt < nrt) {  // uniform
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) red[wv][ct][lane] = acc[rt][ct];
        __syncthreads();
        if (wv < NCT) {  // wave ct adds column tile ct
          const int ct = wv;
          f32x4 v = red[0][ct][lane];
          for (int q = 1; q < kLoraWaves; ++q) v += red[q][ct][lane];
          // D lane (j, g): column 16 ct + j, rows 16 rt + 4 g + r
          const int n = 16 * ct + i16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = mb + 16 * rt + 4 * g + r;
            if (row < r1 && n < a.N) a.t[(int64_t)row * a.ldt + n] = v[r];
          }
        }
        __syncthreads();
      }
    }
  }
}

hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  if (a.N < 8 || a.N > 64 || a.N % 8 || a.K % 32 || a.K <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.n_groups), block(64 * kLoraWaves);
  switch ((a.N + 15) / 16) {
    case 1: hipLaunchKernelGGL(lora_a_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(lora_a_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(lora_a_kernel<3>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(lora_a_kernel<4>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Expert-parallel send side ("Serving K3, 01 architecture": expert parallelism with an all-to-all of
// data-dependent sizes; "Kimi K3: architectural innovations", "Compress the expert interface": the
// dispatched payload is the latent). With the experts in contiguous ranges per rank, the dispatched
// (expert-contiguous) rows are already grouped by destination: the send buffer is the routed input
// gathered in that order, and rank i's share is the rows of its expert range.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ src, int64_t row_bytes,
                                                          const uint8_t* __restrict__ src_scales, int64_t scale_bytes,
                                                          const int32_t* __restrict__ perm, int64_t n_rows,
                                                          uint8_t* __restrict__ rows, uint8_t* __restrict__ scales) {
  for (int64_t r = blockIdx.x; r < n_rows; r += gridDim.x) {
    const int64_t from = perm[r];
    const u32x4* s4 = (const u32x4*)(src + from * row_bytes);
    u32x4* d4 = (u32x4*)(rows + r * row_bytes);
    for (int64_t c = threadIdx.x; c < row_bytes / 16; c += 256) d4[c] = s4[c];
    for (int64_t c = threadIdx.x; c < scale_bytes; c += 256) scales[r * scale_bytes + c] = src_scales[from * scale_bytes + c];
  }
}

hipError_t launch_gather_rows(const uint8_t* src, int64_t row_bytes, const uint8_t* src_scales, int64_t scale_bytes,
                              const int32_t* perm, int64_t n_rows, uint8_t* rows, uint8_t* scales, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (row_bytes % 16 || (scale_bytes > 0 && (!src_scales || !scales))) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)std::min<int64_t>(n_rows, 8192);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, s, src, row_bytes, src_scales, scale_bytes, perm,
                     n_rows, rows, scales);
  return hipGetLastError();
}

__global__ void send_counts_kernel(const int32_t* __restrict__ offsets, int n_ranks, int per,
                                   int32_t* __restrict__ send_counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_ranks) send_counts[i] = offsets[(i + 1) * per] - offsets[i * per];
}

hipError_t launch_send_counts(const int32_t* offsets, int n_ranks, int per, int32_t* send_counts, hipStream_t s) {
  if (n_ranks <= 0 || per <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(send_counts_kernel, dim3((unsigned)ceil_div(n_ranks, 64)), dim3(64), 0, s, offsets, n_ranks, per,
                     send_counts);
  return hipGetLastError();
}

// Expert row ranges from received counts: like route_offsets_kernel, with negative counts taken as zero
// and every offset clamped to the rows actually received.
__global__ __launch_bounds__(kRouteThreads) void offsets_clamped_kernel(int E, const int32_t* __restrict__ counts,
                                                                        int64_t limit, int32_t* __restrict__ offsets) {
  __shared__ int64_t part[kRouteThreads];
  const int tid = threadIdx.x;
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int64_t run = 0;
  for (int e = e0; e < e1; ++e) run += max(counts[e], 0);
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t acc = part[tid] - run;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = (int32_t)min(acc, limit);
    acc += max(counts[e], 0);
  }
  if (tid == kRouteThreads - 1) offsets[E] = (int32_t)min(part[kRouteThreads - 1], limit);
}

hipError_t launch_offsets(const int32_t* counts, int E, int64_t limit, int32_t* offsets, hipStream_t s) {
  if (E < 1 || E > kMaxExperts || limit < 0 || limit > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(offsets_clamped_kernel, dim3(1), dim3(kRouteThreads), 0, s, E, counts, limit, offsets);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Plain streaming read (measurement of the HBM read rate a simple kernel reaches): block b reads a
// contiguous range of the buffer once, 256 threads x 16 bytes a load, eight non-temporal loads in
// flight per thread (the way the weight streams of the grouped GEMMs load); the xor of every word is
// folded into one word so that no load is dead.
// ---------------------------------------------------------------------------------------------
constexpr int kStreamBlocks = 256 * 8;
constexpr int kStreamUnroll = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* buf, int64_t per, int64_t bytes, uint32_t* out) {
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t n = min(per, bytes - b0);
  u32 acc = 0;
  if (n > 0) {
    const rsrc_t r = make_rsrc(buf + b0, n);
    const int t16 = threadIdx.x * 16;
    for (int64_t o = 0; o < n; o += 4096 * kStreamUnroll) {
      u32x4 v[kStreamUnroll];
#pragma unroll
      for (int i = 0; i < kStreamUnroll; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o + t16 + 4096 * i, 0, kNT);
#pragma unroll
      for (int i = 0; i < kStreamUnroll; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    }
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= (u32)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(out, acc);
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
  if (bytes <= 0 || bytes % 16 || !buf || !out) return hipErrorInvalidValue;
  // equal contiguous ranges (multiples of 16 bytes, each below 2 GiB for the 32-bit buffer offsets)
  const int64_t per = (ceil_div(ceil_div(bytes, kStreamBlocks), 16)) * 16;
  if (per >= ((int64_t)1 << 31) - 4096 * kStreamUnroll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0, s, (const uint8_t*)buf, per, bytes, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Static device scratch for the entry point that allocates nothing. Each GPU the library runs on holds
// its own copy of the array (allocated when the code object is loaded there) until the process ends.
// Host code never uses the array's name as a device address: its address on each device is looked up
// once, with that device current, and kept.
// ---------------------------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace k3
