// Fused decode attention over the packed 2/4-bit cache.
//
// [paper] "OmniKVQuant: KV Cache Quantization for Omni-LLMs", §1 and Fig. 1(d):
// the query is rotated once per head instead of inverse-rotating every cached
// key, the online softmax follows FlashAttention's order, value accumulators
// stay in the rotated space of each modality, and the inverse value rotations
// are batched across head outputs; no dense FP16 cache is built ([abstract]).
//
// Split-KV: kernel 1 (decode_partial) gives every (sequence, KV head, split of
// consecutive windows) one workgroup of four 64-lane waves, each wave a
// contiguous run of windows; the block merges its waves and writes (running max,
// sum, three per-modality accumulators in rotated space); kernel 2
// (decode_combine) merges the splits with the log-sum-exp rule and applies
// sum_m U_m A_m once per head.
//
// Per 32-token window the wave issues two kinds of matrix-core contraction
// (v_mfma_f32_16x16x32_f16):
//   scores^T [32 tok x 16 col] = codes [32 x d] . Qt [d x 16]
//   acc^T    [d x 16 col]     += levels^T [d x 32 tok] . Pt [32 x 16]
// For the scores the 16 columns are the G <= 8 query heads of the KV head, twice:
// columns 0..7 carry the fp16 "hi" part and 8..15 the "lo" remainder of the fp32
// operand, so each product keeps ~22 significant bits and the two halves add up
// after the contraction (one DPP row rotate).  For the values the 16 columns are
// the heads of two modalities (accumulator A: audio, video; B: text) and the hi
// and lo parts of p * sigma enter as two contractions into the same columns.
//   Key codes enter as fp16 subnormals: masking a stored word leaves
//   code * 2^(bits*p - 24) in each half, exact in fp16 and exact in the f32
//   accumulation; the per-K-step power of two is folded into Qt.
//   Score algebra: score_log2 = Z_h * (q^.m_w + 2^24 * C) with
//   q^ = log2(e) * scale * R q / Z_h (|q^| <= 1, Z_h a power of two),
//   C = sum_c code_c * 2^-24 * (q^_c s_c); the q^.m_w term comes from four extra
//   contractions per window with k_min as the operand.
//   Value levels come from a per-context table of fp16 level pairs indexed by
//   two packed codes (LDS, conflict-free for 2-bit).
//   MXFP4 key metadata ([paper] §3.1 Implementation details: the default format)
//   arrive as per-window records of E2M1 codes and E8M0 block exponents; each wave
//   expands a window's two records into the fp16 k_scale / k_min areas of its LDS
//   slot (v_cvt_scalef32_pk_f16_fp4, exact in fp16's range) before the window's
//   contractions, which are then the same as with fp16 metadata.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "omnikv_internal.h"

namespace omnikv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

// The value operand of token t is x_t = p_t sigma_t, p_t = 2^(s_t - R) with R the running
// reference (log2 units), split into fp16 hi and lo parts.  R follows a bound of
// log2(p_t sigma_t) instead of the score alone, so x stays inside fp16's range whatever the
// value scales are: R moves (and the accumulators are rescaled) only when that bound exceeds
// 2^kXMax, and then so that it becomes 2^kXAfter.  Between moves x < 2^15 (fp16 holds up to
// 65504); right after one the tokens that dominate the sums have x near 2^kXAfter, where
// both fp16 parts are normal numbers and the pair keeps ~22 bits.
constexpr float kXMax = 15.0f;
constexpr float kXAfter = 7.0f;
constexpr uint32_t kHiLimitBits = 0x7800u;  // fp16 2^15 (= 2^kXMax)
typedef uint16_t ushort2_t __attribute__((ext_vector_type(2)));

// Biased exponent field e of the largest of a lane's eight fp16 value scales (two per word):
// every one of them is below 2^(e - 14) (e = 0 for zero and subnormal scales).  Scales are
// non-negative, so their bit patterns order like their values.
__device__ __forceinline__ float scale_exponent_field(const uint32_t (&sgw)[4]) {
  const ushort2_t a = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, sgw[0]), __builtin_bit_cast(ushort2_t, sgw[1]));
  const ushort2_t b = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, sgw[2]), __builtin_bit_cast(ushort2_t, sgw[3]));
  const ushort2_t c = __builtin_elementwise_max(a, b);
  const uint32_t m = max(static_cast<uint32_t>(c.x), static_cast<uint32_t>(c.y));
  return static_cast<float>((m >> 10) & 31u);
}

__device__ __forceinline__ float f16_value(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float4_t mfma16(uint4_t a, uint4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// value of lane (l ^ 8) within each row of 16 lanes (DPP row_ror:8).  Every lane reads a
// valid source lane, so the move needs no prior value (a zero-filled destination would cost
// one more instruction per move).
__device__ __forceinline__ float row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
}

// Wave votes straight from the lane mask of the predicate (the __all / __any forms turn the
// mask into a 0/1 per lane and compare that again).  The predicate should be one comparison:
// a combination of several is materialized per lane before the vote.
__device__ __forceinline__ bool wave_all(bool p) {
  return __builtin_amdgcn_ballot_w64(p) == __builtin_amdgcn_read_exec();
}
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Cross-half lane swaps.  Written in asm: the compiler's combine of the
// permlane{16,32}_swap builtins can replace the second result by the first
// (as if the operand were the same in every lane), which drops the lanes the
// swap brings in.  Each asm swaps two registers in place and touches no memory.
// The s_nop pairs give the wait states a VALU write needs before a permlane
// reads the register, and a permlane result before the next VALU reads it
// (the hazard recognizer does not look inside asm).
//   swap32(a, b): lanes 32..63 of a <-> lanes 0..31 of b
//   swap16(a, b): odd 16-lane rows of a <-> even rows of b
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// reduce over the four 16-lane groups holding the same column (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);  // a = lower half in both halves, b = upper half in both halves
  x = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float group_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// value of lane l ^ (1 << K) within each 16-lane row (K = 0 .. 3), by DPP moves; each
// move reads a valid source lane for every lane it writes
template <int K>
__device__ __forceinline__ float lane_xor_row(float x) {
  const int v = __builtin_bit_cast(int, x);
  if constexpr (K == 0) {  // quad_perm [1, 0, 3, 2]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  } else if constexpr (K == 1) {  // quad_perm [2, 3, 0, 1]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  } else if constexpr (K == 2) {
    // lanes 0-3 and 8-11 of a row read lane + 4 (row_shl:4), lanes 4-7 and 12-15 lane - 4
    // (row_shr:4); the bank mask picks which lanes each move writes
    const int lo = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0x5, false);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(lo, v, 0x114, 0xF, 0xA, false));
  } else {  // row_ror:8
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));
  }
}

// One radix-2 stage of the Walsh-Hadamard transform across the lanes of a wave, partner
// lane l ^ ST: the lane with that bit clear takes own + partner, the other partner - own.
template <int ST>
__device__ __forceinline__ float wht_lane_stage(float z, int lane) {
  if constexpr (ST < 16) {
    constexpr int K = ST == 1 ? 0 : (ST == 2 ? 1 : (ST == 4 ? 2 : 3));
    const float p = lane_xor_row<K>(z);
    return (lane & ST) ? p - z : z + p;
  } else {
    static_assert(ST == 16 || ST == 32, "lane stages");
    uint32_t a = __builtin_bit_cast(uint32_t, z), b = a;
    if constexpr (ST == 16) swap16(a, b);
    else swap32(a, b);
    // a: the value of the lane with the bit clear, b: of the lane with it set
    const float fa = __builtin_bit_cast(float, a), fb = __builtin_bit_cast(float, b);
    return (lane & ST) ? fa - fb : fa + fb;
  }
}

// 2^x by the hardware instruction (results below 2^-126 flush to zero; the softmax
// weights it produces are relative to a running max, so those are negligible)
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// fp16 pair (lo half, hi half) = (fp16(p0 s0 - c0), fp16(p1 s1 - c1)): each half one fused
// multiply-add of an fp32 by an fp16 (both halves of s) minus an fp16 (halves of c),
// rounded once to fp16 (v_fma_mix{lo,hi}_f16).  The leading wait state covers an operand
// just written by a transcendental instruction (the hazard recognizer does not look
// inside asm).
__device__ __forceinline__ uint32_t mix_pair(float p0, float p1, uint32_t s, uint32_t c) {
  uint32_t d;  // both halves are written here, so its earlier contents do not matter
  asm("s_nop 0\n\t"
      "v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %0, %4, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
      : "=&v"(d)
      : "v"(p0), "v"(s), "v"(c), "v"(p1));
  return d;
}

// The same for the four dwords of a lane's eight probabilities (dword q: p[2q], p[2q + 1]
// with the halves of s[q] and c[q]), in one block with one wait state.
__device__ __forceinline__ void mix_quad(const float (&p)[8], const uint32_t (&s)[4], const uint32_t (&c)[4],
                                         uint32_t (&d)[4]) {
  asm("s_nop 0\n\t"
      "v_fma_mixlo_f16 %0, %4, %12, -%16 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %0, %5, %12, -%16 op_sel:[0,1,1] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixlo_f16 %1, %6, %13, -%17 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %1, %7, %13, -%17 op_sel:[0,1,1] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixlo_f16 %2, %8, %14, -%18 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %2, %9, %14, -%18 op_sel:[0,1,1] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixlo_f16 %3, %10, %15, -%19 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %3, %11, %15, -%19 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]),
        "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]), "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]));
}

template <int D>
struct RhtConst;
template <>
struct RhtConst<64> {
  static constexpr float value = 0.125f;
};
template <>
struct RhtConst<128> {
  static constexpr float value = 0.08838834764831845f;
};

// Key operand geometry (window-block layout of include/omnikv.h).
template <int D, int KB>
struct KeyOp {
  static constexpr int words = D * KB / 64;  // per lane
  // effective slot of K-step s after the shift: the operand holds code * 2^(KB*peff - 24)
  __device__ static constexpr int peff(int s) {
    return (D == 128 && KB == 4) ? (s & 1) : s;
  }
  __device__ static constexpr int word(int tau, int s, int i) {
    if (D == 128 && KB == 2) return i;
    if (D == 128 && KB == 4) return 4 * tau + i;
    if (D == 64 && KB == 2) return i & 1;
    return i;
  }
  __device__ static constexpr int shift(int tau, int s, int i) {
    if (D == 128 && KB == 2) return 8 * tau;
    if (D == 128 && KB == 4) return 8 * (s >> 1);
    if (D == 64 && KB == 2) return 8 * (i >> 1) + 4 * tau;
    return 8 * tau;
  }
  __device__ static constexpr uint32_t mask(int s) {
    return (((1u << KB) - 1u) * 0x00010001u) << (KB * peff(s));
  }
};

struct PartialArgs {
  const float* q;
  const int32_t* seq_lens;
  const uint32_t* k_codes;
  const uint16_t* k_min;
  const uint16_t* k_scale;
  const uint32_t* v_codes;
  const uint16_t* v_scale;
  const uint8_t* modality;
  const float* signs;
  const uint32_t* pair_table;
  int hq, hkv, group, modalities;
  int64_t t_cap;
  int64_t max_len;   // host bound of seq_lens; device lengths are clamped to it
  float scale_log2;  // softmax scale * log2(e)
  int wpw, splits;   // windows per wave; splits (= workgroups) per (sequence, KV head)
  int split_old, wpw_young;  // splits [split_old, splits) take wpw_young windows per wave
  float2* ws_ml;     // [unit][split][8] (max, sum) in log2 units
  uint32_t* ws_mask; // [unit][split] modalities present
  float* ws_acc;     // [unit][split][M][8][D]
  int stream;        // 1: attend over the value-packed prefix of each stream (the rest is recent)
  // streamed sequences: workgroup `splits` of each unit scores the recent tokens instead
  const void* k_ring;  // [B][ring_cap][Hkv][d], bf16 or fp32
  const void* v_ring;
  int ring_f32, ring_cap;
  float2* tail_ml;   // [unit][8] (max, sum) of the recent tokens, log2 units
  float* tail_o;     // [unit][8][D] their value sum in the original space, relative to the max
};

// ---------------------------------------------------------------------------------------
// Window staging.  Each wave owns a ring of LDS slots; a slot holds everything one
// 32-token window needs: [key block | value block | k_scale | k_min | v_scale | tags],
// and with MXFP4 key metadata the two raw records after them (k_scale, k_min), which
// the wave expands into the fp16 k_scale and k_min areas before the window's visit.
// Slots are filled by asynchronous global->LDS copies (global_load_lds_dwordx4, 16 bytes
// per lane), ring depth - 1 windows ahead of the one being computed, so no registers are
// held by loads in flight.  The copies are tracked by the vmcnt counter only; the waits
// before reading a slot are explicit.
constexpr int kWaves = 4;  // waves per workgroup; each owns its own consecutive windows

template <int D, int KB, int VB, bool MX>
struct Slot {
  static constexpr int KBYTES = 4 * D * KB;  // 32 tokens x D codes x KB bits
  static constexpr int VBYTES = 4 * D * VB;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = KBYTES;
  static constexpr int OFF_S = KBYTES + VBYTES;      // k_scale, 2 D bytes (fp16)
  static constexpr int OFF_M = OFF_S + 2 * D;        // k_min, 2 D bytes (fp16)
  static constexpr int OFF_SIG = OFF_M + 2 * D;      // v_scale of the 32 tokens, 64 bytes
  static constexpr int OFF_TAG = OFF_SIG + 64;       // modality of the 32 tokens, 32 bytes
  static constexpr int MXR = mx_record_bytes(D);     // MXFP4: one record
  static constexpr int OFF_RAW = OFF_TAG + 32;       // MXFP4: k_scale record, then k_min's
  static constexpr int END = MX ? OFF_RAW + 2 * MXR : OFF_TAG + 32;
  static constexpr int BYTES = (END + 127) / 128 * 128;
  static constexpr int NK = (KBYTES + 1023) / 1024;  // copies of the key block
  static constexpr int NV = (VBYTES + 1023) / 1024;
  // the metadata copy: one 16-byte piece per lane, in lane order from OFF_COPY
  static constexpr int OFF_COPY = MX ? OFF_SIG : OFF_S;
  static constexpr int MISC_LANES = (END - OFF_COPY) / 16;
  static constexpr int COPIES = NK + NV + 1;          // copy instructions per window
  static_assert(OFF_RAW % 16 == 0 && MXR % 16 == 0, "copy pieces");
};

// One 16-byte-per-lane global->LDS copy (lane l writes lds_addr + 16 l).  Issued in asm so
// the compiler's wait insertion does not see it: it cannot tell ring slots apart and would
// drain every copy in flight before each slot read.  The copy writes no VGPR; its only
// consumers are the slot reads that follow an explicit wait_vmcnt.
// The copy takes its LDS base from M0, which the asm sets and declares clobbered (the
// compiler re-establishes M0 itself wherever it relies on it).
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_addr)
      : "memory", "m0");
}

// The same copy from a wave-uniform 64-bit base plus a 32-bit per-lane byte offset (the
// scalar-base form of the global address), which keeps the address math in 32 bits.
__device__ __forceinline__ void copy16_to_lds_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory", "m0");
}

// One 4-byte global->LDS copy per active lane (lane l writes lds_addr + 4 l); the same
// M0 handling as above.
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(lds_addr)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` groups of L copies are still in flight (ahead <= A).
template <int L, int A>
__device__ __forceinline__ void wait_groups(int ahead) {
  if constexpr (A <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) wait_vmcnt<A * L>();
    else wait_groups<L, A - 1>(ahead);
  }
}

// Ring depth: the deepest of 4, 3, 2 slots per wave that keeps kBlocksPerCU workgroups per
// CU within the 160 KB of LDS (ring + rotated queries + small tables); deeper rings
// measured slower.  Two workgroups per CU (two waves per SIMD) measured as fast as three
// and leave each wave registers for its operand constants.
constexpr int kBlocksPerCU = 2;
// Dynamic LDS: the ring, filled by the asynchronous copies.  Before the visits a wave's
// last ring slot (not filled before the first visit) stages its two query heads, the
// signs of D, the sequence's length and (wave 0) the level-pair table; after them the
// whole region holds every wave's per-modality accumulators for the block merge.
template <int D, int KB, int VB, bool MX>
struct Lds {
  static constexpr int QRAW = 2 * D * 4;         // staging: two heads' queries, fp32
  static constexpr int SGN = D * 4;              // then the signs of D, fp32
  static constexpr int LEN = QRAW + SGN;         // then the length (4 bytes, 16 reserved)
  static constexpr int TAB_OFF = LEN + 16;       // then the level-pair table
  static constexpr int TAB = 4 << (2 * VB);
  static constexpr int MERGE = kWaves * kMaxModalities * kMaxGroup * (D + 16) * 4;  // padded rows
  static constexpr int STATIC = kMaxGroup * D * 4 + TAB + 1024;  // q_lds, the table, small arrays
  static constexpr int dyn(int ring) {
    const int r = kWaves * ring * Slot<D, KB, VB, MX>::BYTES;
    return r > MERGE ? r : MERGE;
  }
  static constexpr bool fits(int ring) { return dyn(ring) + STATIC <= 160 * 1024 / kBlocksPerCU; }
  static constexpr int RING = fits(4) ? 4 : (fits(3) ? 3 : 2);
  static constexpr int RING_BYTES = kWaves * RING * Slot<D, KB, VB, MX>::BYTES;
  static constexpr int DYN = dyn(RING);
  static_assert(fits(RING), "LDS budget");
  static_assert(TAB_OFF + TAB <= Slot<D, KB, VB, MX>::BYTES, "staging must fit in one slot");
};

// The recent tokens [T0, n) of a streamed sequence (T0 = max(value-packed length, n -
// ring_cap)), for the 8 query heads of one KV head at once, by one workgroup:
//   scores in log2 units: a token below the key-packed length from its packed key with the
//   rotated query (q_rot, already scaled by c_d and the softmax scale), a later one from its
//   stored key with the query itself;
//   then per head the max, the sum of 2^(s - max) and the value sum in the original space.
// scratch: [8][D] original queries, then [8][kMaxRingCap] scores (dynamic LDS).
template <int D, int KB, bool MX>
__device__ void stream_tail(const PartialArgs& a, const float (*q_rot)[D], float* scratch, int unit, int b,
                            int kvh, int n) {
  constexpr int T = kWaves * 64;
  constexpr int PER_LANE = D * KB / 64;                     // words per block lane
  constexpr int NW = (D == 128 && KB == 4) ? 4 : PER_LANE;  // words of one token half
  constexpr int CPT = D / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kp = static_cast<int>(stream_key_packed(n));
  const int T0 = max(static_cast<int>(stream_value_packed(n)), n - a.ring_cap);
  const int nt = max(0, n - T0);
  float* qo = scratch;                 // [8][D]
  float* sc = scratch + kMaxGroup * D; // [8][kMaxRingCap]
  for (int i = tid; i < kMaxGroup * D; i += T) {
    const int hh = i / D;
    qo[i] = hh < a.group ? a.q[(static_cast<size_t>(b) * a.hq + kvh * a.group + hh) * D + i % D] : 0.0f;
  }
  __syncthreads();
  // scores: eight threads per token, CPT consecutive channels each (one channel group g of
  // the key window block, whose lane words 16 g + rho hold their codes), summed over the
  // eight by row moves
  const int64_t nwin_cap = a.t_cap / kWindow;
  const int sub = tid & 7, c0 = sub * CPT;
  const int g = c0 / (D / 4), sh2 = (c0 % (D / 4)) / 8;  // group, first 8-channel step
  for (int j0 = 0; j0 < nt; j0 += T / 8) {
    const int j = j0 + (tid >> 3);
    float acc[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) acc[hh] = 0.0f;
    if (j < nt) {
      const int t = T0 + j;
      if (t < kp) {
        const size_t wb = static_cast<size_t>(unit) * nwin_cap + t / kWindow;
        const int tt = t % kWindow, tau = tt >> 4, rho = tt & 15;
        const uint32_t* wp = a.k_codes + wb * (D * KB) + (16 * g + rho) * PER_LANE + ((D == 128 && KB == 4) ? 4 * tau : 0);
        uint32_t w[NW];
#pragma unroll
        for (int x = 0; x < NW; ++x) w[x] = wp[x];
        float mv_[CPT], sv_[CPT];
        if constexpr (!MX) {
          uint32_t mw[CPT / 2], sw[CPT / 2];
#pragma unroll
          for (int x = 0; x < CPT; x += 8) {
            const uint4 m8 = *reinterpret_cast<const uint4*>(a.k_min + wb * D + c0 + x);
            const uint4 s8 = *reinterpret_cast<const uint4*>(a.k_scale + wb * D + c0 + x);
            mw[x / 2] = m8.x; mw[x / 2 + 1] = m8.y; mw[x / 2 + 2] = m8.z; mw[x / 2 + 3] = m8.w;
            sw[x / 2] = s8.x; sw[x / 2 + 1] = s8.y; sw[x / 2 + 2] = s8.z; sw[x / 2 + 3] = s8.w;
          }
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc) {
            mv_[cc] = f16_value(static_cast<uint16_t>(mw[cc >> 1] >> (16 * (cc & 1))));
            sv_[cc] = f16_value(static_cast<uint16_t>(sw[cc >> 1] >> (16 * (cc & 1))));
          }
        } else {
          // MXFP4 records: channels c0 .. c0 + CPT - 1 lie in one 32-channel block
          constexpr int R = mx_record_bytes(D);
          const uint8_t* rm = reinterpret_cast<const uint8_t*>(a.k_min) + wb * R;
          const uint8_t* rs = reinterpret_cast<const uint8_t*>(a.k_scale) + wb * R;
          const int em = static_cast<int>(rm[D / 2 + c0 / 32]) - 127;
          const int es = static_cast<int>(rs[D / 2 + c0 / 32]) - 127;
          uint32_t nm[CPT / 8], ns[CPT / 8];
#pragma unroll
          for (int x = 0; x < CPT / 8; ++x) {
            nm[x] = *reinterpret_cast<const uint32_t*>(rm + c0 / 2 + 4 * x);
            ns[x] = *reinterpret_cast<const uint32_t*>(rs + c0 / 2 + 4 * x);
          }
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc) {
            mv_[cc] = mx_decode((nm[cc >> 3] >> (4 * (cc & 7))) & 15u, em);
            sv_[cc] = mx_decode((ns[cc >> 3] >> (4 * (cc & 7))) & 15u, es);
          }
        }
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          const int jj = cc & 7, i = jj >> 1, e = jj & 1, s8i = sh2 + (cc >> 3);
          uint32_t word, bit;
          if (D == 128 && KB == 2) { word = w[i]; bit = 16 * e + 2 * (4 * tau + s8i); }
          else if (D == 128) { word = w[i]; bit = 16 * e + 4 * s8i; }
          else if (KB == 2) { word = w[i & 1]; bit = 16 * e + 2 * (4 * (i >> 1) + 2 * tau + s8i); }
          else { word = w[i]; bit = 16 * e + 4 * (2 * tau + s8i); }
          const float code = static_cast<float>((word >> bit) & ((1u << KB) - 1u));
          const float kval = mv_[cc] + sv_[cc] * code;
#pragma unroll
          for (int hh = 0; hh < kMaxGroup; ++hh) acc[hh] = fmaf(q_rot[hh][c0 + cc], kval, acc[hh]);
        }
      } else {
        const size_t row = ((static_cast<size_t>(b) * a.ring_cap + t % a.ring_cap) * a.hkv + kvh) * D + c0;
        float kv[CPT];
        if (a.ring_f32) {
#pragma unroll
          for (int x = 0; x < CPT; x += 4) {
            const float4 k4 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.k_ring) + row + x);
            kv[x] = k4.x; kv[x + 1] = k4.y; kv[x + 2] = k4.z; kv[x + 3] = k4.w;
          }
        } else {
#pragma unroll
          for (int x = 0; x < CPT; x += 8) {
            const uint4 k8 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_ring) + row + x);
            const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
            for (int y = 0; y < 8; ++y) kv[x + y] = __uint_as_float((y & 1) ? (kw[y >> 1] & 0xFFFF0000u) : (kw[y >> 1] << 16));
          }
        }
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
          for (int hh = 0; hh < kMaxGroup; ++hh) acc[hh] = fmaf(qo[hh * D + c0 + cc], kv[cc], acc[hh]);
#pragma unroll
        for (int hh = 0; hh < kMaxGroup; ++hh) acc[hh] *= a.scale_log2;
      }
    }
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      acc[hh] += __shfl_xor(acc[hh], 1, 64);
      acc[hh] += __shfl_xor(acc[hh], 2, 64);
      acc[hh] += __shfl_xor(acc[hh], 4, 64);
    }
    if (j < nt && sub == 0) {
#pragma unroll
      for (int hh = 0; hh < kMaxGroup; ++hh) sc[hh * kMaxRingCap + j] = acc[hh];
    }
  }
  __syncthreads();
  // per head (wave w: heads 2w, 2w + 1): max, probabilities in place, their sum
  __shared__ float2 tml[kMaxGroup];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int hh = 2 * wave + x;
    float m = -INFINITY;
    for (int j = lane; j < nt; j += 64) m = fmaxf(m, sc[hh * kMaxRingCap + j]);
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1) m = fmaxf(m, __shfl_xor(m, st, 64));
    float l = 0.0f;
    for (int j = lane; j < nt; j += 64) {
      const float p = exp2f(sc[hh * kMaxRingCap + j] - m);
      sc[hh * kMaxRingCap + j] = p;
      l += p;
    }
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1) l += __shfl_xor(l, st, 64);
    if (lane == 0) tml[hh] = make_float2(m, nt > 0 ? l : 0.0f);
  }
  __syncthreads();
  // value sums in the original space: thread (c, head quarter), 8 / (T / D) heads each
  constexpr int HPT = kMaxGroup * D / T;
  const int c = tid % D, hq0 = (tid / D) * HPT;
  float o[HPT];
#pragma unroll
  for (int x = 0; x < HPT; ++x) o[x] = 0.0f;
  // 32 tokens' values are loaded together (past the last token: the last token again, with
  // weight zero), without branches, so the loads are in flight at once
  constexpr int VBT = 32;
  const size_t vrow0 = (static_cast<size_t>(b) * a.ring_cap * a.hkv + kvh) * D + c;
  const size_t vstride = static_cast<size_t>(a.hkv) * D;  // elements per ring row
  for (int j0 = 0; j0 < nt; j0 += VBT) {
    float vv[VBT];
    if (a.ring_f32) {
#pragma unroll
      for (int y = 0; y < VBT; ++y) {
        const int t = T0 + min(j0 + y, nt - 1);
        vv[y] = static_cast<const float*>(a.v_ring)[vrow0 + static_cast<size_t>(t % a.ring_cap) * vstride];
      }
    } else {
#pragma unroll
      for (int y = 0; y < VBT; ++y) {
        const int t = T0 + min(j0 + y, nt - 1);
        vv[y] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.v_ring)[vrow0 + static_cast<size_t>(t % a.ring_cap) * vstride]) << 16);
      }
    }
#pragma unroll
    for (int y = 0; y < VBT; ++y) {
      const bool ok = j0 + y < nt;
#pragma unroll
      for (int x = 0; x < HPT; ++x) o[x] = fmaf(ok ? sc[(hq0 + x) * kMaxRingCap + j0 + y] : 0.0f, vv[y], o[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < HPT; ++x) a.tail_o[(static_cast<size_t>(unit) * kMaxGroup + hq0 + x) * D + c] = o[x];
  if (tid < kMaxGroup) a.tail_ml[static_cast<size_t>(unit) * kMaxGroup + tid] = tml[tid];
}

template <int D, int KB, int VB, bool MX>
__global__ __launch_bounds__(kWaves * 64, kBlocksPerCU) void decode_partial_kernel(PartialArgs a) {
  using SG = Slot<D, KB, VB, MX>;
  using KO = KeyOp<D, KB>;
  constexpr int RING = Lds<D, KB, VB, MX>::RING;
  constexpr int NC = D / 64;        // channels per lane in the query rotation
  constexpr int NS = D / 32;        // K-steps of the score contraction
  constexpr int NU = D / 16;        // channel tiles of the value contraction
  constexpr int KW = KO::words;     // key words per lane
  constexpr int VW = D * VB / 64;   // value words per lane
  constexpr int PPW = 16 / VB;      // value code pairs per word
  constexpr uint32_t PMASK = (1u << (2 * VB)) - 1u;
  constexpr int L = SG::COPIES;
  using LY = Lds<D, KB, VB, MX>;

  // Dynamic LDS (layout in Lds).  Only the asm copies write the ring and the staging
  // areas, and a static LDS array that no visible code stores to would let the optimizer
  // treat its contents as undefined and fold the reads.
  extern __shared__ __attribute__((aligned(16))) uint8_t ring_mem[];
  __shared__ __attribute__((aligned(16))) float q_lds[kMaxGroup][D];
  __shared__ float zmax_lds[kMaxGroup];
  __shared__ uint32_t vtab[1 << (2 * VB)];
  // 2-bit values: the level quads of a code byte (its low and high nibbles' level pairs)
  __shared__ __attribute__((aligned(8))) uint2 vquad[VB == 2 ? 256 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int unit = blockIdx.x;                     // b * hkv + kvh
  const int split = blockIdx.y;
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int h0 = 2 * wave;                         // this wave's two query heads
  // this wave's run of windows: splits below split_old (dispatched first, so older on
  // their SIMDs) take wpw windows per wave, the later ones wpw_young
  const int wbeg = split < a.split_old ? (split * kWaves + wave) * a.wpw
                                       : a.split_old * kWaves * a.wpw + ((split - a.split_old) * kWaves + wave) * a.wpw_young;
  const int my_wpw = split < a.split_old ? a.wpw : a.wpw_young;

  // ---- first copies, before anything waits for memory: this wave's two heads of the
  // query, the signs of D, the level-pair table (wave 0), then the first windows.  The
  // windows are bounded by the host's max_len, as the sequence's own length is not known
  // yet; copies past it are drained before the ring is reused.
  const auto lds_addr = [&](int off) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring_mem + off)));
  };
  const int stage_off = (wave * RING + RING - 1) * SG::BYTES;  // this wave's last slot
  {
    constexpr int qlanes = LY::QRAW / 16, slanes = LY::SGN / 16, tlanes = LY::TAB / 16;
    if (lane < qlanes) {
      const int j = (16 * lane) / (4 * D);  // head h0 + j; heads past the group copy head 0 (zeroed later)
      const int hh = (h0 + j < a.group) ? h0 + j : 0;
      const float* src = a.q + (static_cast<size_t>(b) * a.hq + kvh * a.group + hh) * D + (4 * lane) % D;
      copy16_to_lds(src, lds_addr(stage_off));
    }
    if (lane < slanes) copy16_to_lds(a.signs + 4 * lane, lds_addr(stage_off + LY::QRAW));
    if (lane == 0) copy4_to_lds(a.seq_lens + b, lds_addr(stage_off + LY::LEN));
    if (wave == 0 && lane < tlanes) copy16_to_lds(a.pair_table + 4 * lane, lds_addr(stage_off + LY::TAB_OFF));
  }
  const int n = lane & 15, g = lane >> 4, h = n & 7, part = n >> 3;
  const int64_t nwin_cap = a.t_cap / kWindow;
  const size_t unit_win = static_cast<size_t>(unit) * nwin_cap;

  // ---- per-lane copy descriptors: source = base + window * stride (bytes)
  // key and value blocks: wave-uniform base of this unit + 32-bit offsets (a unit's blocks
  // span at most t_cap / 32 windows of a few KB)
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_codes) + unit_win * SG::KBYTES;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_codes) + unit_win * SG::VBYTES;
  const uint8_t* mbase = nullptr;
  uint32_t mstride = 0;
  if constexpr (MX) {
    // [v_scale: 4 pieces | tags: 2 | k_scale record | k_min record]
    constexpr int RP = SG::MXR / 16;
    if (lane < 4) {
      mbase = reinterpret_cast<const uint8_t*>(a.v_scale) + static_cast<size_t>(unit) * a.t_cap * 2 + 16 * lane;
      mstride = 64;
    } else if (lane < 6) {
      mbase = a.modality + static_cast<size_t>(b) * a.t_cap + 16 * (lane - 4);
      mstride = 32;
    } else if (lane < 6 + RP) {
      mbase = reinterpret_cast<const uint8_t*>(a.k_scale) + unit_win * SG::MXR + 16 * (lane - 6);
      mstride = SG::MXR;
    } else {
      mbase = reinterpret_cast<const uint8_t*>(a.k_min) + unit_win * SG::MXR + 16 * (lane - 6 - RP);
      mstride = SG::MXR;
    }
  } else {
    const int l0 = D / 8, l1 = D / 4, l2 = D / 4 + 4;
    if (lane < l0) {
      mbase = reinterpret_cast<const uint8_t*>(a.k_scale) + unit_win * (2 * D) + 16 * lane;
      mstride = 2 * D;
    } else if (lane < l1) {
      mbase = reinterpret_cast<const uint8_t*>(a.k_min) + unit_win * (2 * D) + 16 * (lane - l0);
      mstride = 2 * D;
    } else if (lane < l2) {
      mbase = reinterpret_cast<const uint8_t*>(a.v_scale) + static_cast<size_t>(unit) * a.t_cap * 2 + 16 * (lane - l1);
      mstride = 64;
    } else {
      mbase = a.modality + static_cast<size_t>(b) * a.t_cap + 16 * (lane - l2);
      mstride = 32;
    }
  }
  // Ring slots as byte offsets from this wave's first slot; the slot to fill next and the
  // metadata copy's per-lane source advance by one slot and one window at each issue.
  constexpr uint32_t RING_SPAN = RING * SG::BYTES;
  const uint32_t ring_lds = lds_addr(wave * RING * SG::BYTES);
  uint32_t fill = 0;
  auto next_slot = [](uint32_t off) { return off + SG::BYTES == RING_SPAN ? 0u : off + SG::BYTES; };
  const uint8_t* mptr = mbase + static_cast<size_t>(wbeg) * mstride;
  auto issue = [&](int w) {
    const uint32_t dst = ring_lds + fill;
#pragma unroll
    for (int x = 0; x < SG::NK; ++x)
      if (1024 * x + 16 * lane < SG::KBYTES)
        copy16_to_lds_sbase(kbase, static_cast<uint32_t>(w * SG::KBYTES + 1024 * x + 16 * lane), dst + SG::OFF_K + 1024 * x);
#pragma unroll
    for (int x = 0; x < SG::NV; ++x)
      if (1024 * x + 16 * lane < SG::VBYTES)
        copy16_to_lds_sbase(vbase, static_cast<uint32_t>(w * SG::VBYTES + 1024 * x + 16 * lane), dst + SG::OFF_V + 1024 * x);
    if (lane < SG::MISC_LANES) copy16_to_lds(mptr, dst + SG::OFF_COPY);
    mptr += mstride;
    fill = next_slot(fill);
  };

  // ---- visit order: the wave's windows in order, each visited once whatever modalities
  // it holds.  Visit i (window wbeg + i) goes to slot i % RING once visit i - RING has
  // been computed; the first copies go out before the query set-up, which hides their
  // latency.
  int issued = 0;
  auto issue_upto = [&](int lim) {
    for (; issued < lim; ++issued) issue(wbeg + issued);
  };
  {
    const int64_t bound = a.stream ? stream_value_packed(a.max_len) : a.max_len;
    const int nwin_bound = static_cast<int>((bound + kWindow - 1) / kWindow);
    issue_upto(min(max(0, min(nwin_bound, wbeg + my_wpw) - wbeg), RING - 1));
  }

  // ---- the staging copies (issued before any window's) have landed: the sequence's
  // length (clamped to the host bound), this wave's visits, the queries of its two heads
  wait_groups<L, RING - 1>(issued);
  int len = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(ring_mem + stage_off + LY::LEN));
  if (wave == 0) {  // the table goes to its own array (read by every wave after the barrier below)
    const uint32_t* t = reinterpret_cast<const uint32_t*>(ring_mem + stage_off + LY::TAB_OFF);
    for (int i = lane; i < (1 << (2 * VB)); i += 64) vtab[i] = t[i];
  }
  len = static_cast<int>(min<int64_t>(max(len, 0), a.max_len));
  const int len_streamed = len;
  if (a.stream) len = stream_value_packed(len);
  const int nwin = (len + kWindow - 1) / kWindow;
  const int wend = min(nwin, wbeg + my_wpw);
  const int nw = max(0, wend - wbeg);
  float qv[2][NC];
  {
    const float* qraw = reinterpret_cast<const float*>(ring_mem + stage_off);
    const float* sgn = reinterpret_cast<const float*>(ring_mem + stage_off + LY::QRAW);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = h0 + j < a.group;
#pragma unroll
      for (int c = 0; c < NC; ++c) qv[j][c] = qraw[j * D + lane + 64 * c] * (ok ? sgn[lane + 64 * c] : 0.0f);
    }
  }

  // ---- query rotation q' = c_d H D q (two heads per wave), scaled to log2 units.  The
  // butterflies across lanes are DPP moves and lane swaps (register to register), both
  // heads' stages side by side.
  float z[2][NC];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < NC; ++c) z[j][c] = qv[j][c];
  auto wht_stage = [&](auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < NC; ++c) z[j][c] = wht_lane_stage<ST>(z[j][c], lane);
  };
  wht_stage(std::integral_constant<int, 1>{});
  wht_stage(std::integral_constant<int, 2>{});
  wht_stage(std::integral_constant<int, 4>{});
  wht_stage(std::integral_constant<int, 8>{});
  wht_stage(std::integral_constant<int, 16>{});
  wht_stage(std::integral_constant<int, 32>{});
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (NC == 2) {
      const float x0 = z[j][0] + z[j][1], x1 = z[j][0] - z[j][1];
      z[j][0] = x0;
      z[j][1] = x1;
    }
    float am = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      z[j][c] = z[j][c] * RhtConst<D>::value * a.scale_log2;
      q_lds[h0 + j][lane + 64 * c] = z[j][c];
      am = fmaxf(am, fabsf(z[j][c]));
    }
    am = fmaxf(am, lane_xor_row<0>(am));
    am = fmaxf(am, lane_xor_row<1>(am));
    am = fmaxf(am, lane_xor_row<2>(am));
    am = fmaxf(am, lane_xor_row<3>(am));
    am = group_max(am);
    if (lane == 0) zmax_lds[h0 + j] = am;
  }
  __syncthreads();

  // ---- streamed sequences: the extra workgroup of the unit takes the recent tokens (it
  // reads the rotated queries from q_lds, before the operand tables below replace them)
  if (a.stream && split == a.splits) {
    // the split workgroups sharing this CU raise their priority while they start: this short
    // one takes the highest too, or it would only get their leftover issue slots
    __builtin_amdgcn_s_setprio(3);
    stream_tail<D, KB, MX>(a, q_lds, reinterpret_cast<float*>(ring_mem), unit, b, kvh, len_streamed);
    return;
  }

  // Z_h: power of two with |q'/Z_h| <= 1
  int zexp = 0;
  {
    const float zm = zmax_lds[h];
    if (zm > 0.0f) (void)frexpf(zm, &zexp);
  }
  const float zh = ldexpf(1.0f, zexp);
  const float zfac = ldexpf(1.0f, zexp + 24);

  // ---- operand constants.  Lane (n, g) feeds column n: head h, part hi (0) or lo (1);
  // K-step s, dword i hold channels c0, c0 + 1 with c0 = g*D/4 + 8 s + 2 i.
  //   alpha/beta/gamma: score operand  fp16 split (th, tl) of (q^ s) scaled by 2^-(KB*peff(s)):
  //                     alpha = th, beta = th (part 1) or 0, gamma = tl (part 1) or 0
  //   bqa:              k_min operand  fp16 split (qh, ql) of q^: qh (part 0) or ql (part 1)
  // with q^ = q'/Z_h.  They depend on (head, channel) only, so the block builds four
  // [head][D] fp16 tables once (a few elements per thread) and every lane loads its rows:
  // th and tl over q_lds, qh and ql in the staging slots of waves 0 and 1 (free until the
  // visits begin).
  constexpr int PER_T = kMaxGroup * D / (kWaves * 64);
  static_assert(PER_T * kWaves * 64 == kMaxGroup * D, "table elements per thread");
  static_assert(2 * kMaxGroup * D * 2 <= kMaxGroup * D * 4, "th and tl tables fit over q_lds");
  static_assert(kMaxGroup * D * 2 <= SG::BYTES, "a qh or ql table fits in a staging slot");
  _Float16 tv[4][PER_T];
#pragma unroll
  for (int x = 0; x < PER_T; ++x) {
    const int idx = tid + x * kWaves * 64, hh = idx / D, c = idx % D;
    const int s = (c % (D / 4)) / 8;
    int ze = 0;
    const float zm = zmax_lds[hh];
    if (zm > 0.0f) (void)frexpf(zm, &ze);
    const float qh = q_lds[hh][c] * ldexpf(1.0f, -ze);                  // |qh| <= 1
    const float qt = qh * ldexpf(1.0f, -KB * KO::peff(s));               // exact scaling
    const _Float16 th = static_cast<_Float16>(qt);
    const _Float16 hq = static_cast<_Float16>(qh);
    tv[0][x] = th;
    tv[1][x] = static_cast<_Float16>(qt - static_cast<float>(th));
    tv[2][x] = hq;
    tv[3][x] = static_cast<_Float16>(qh - static_cast<float>(hq));
  }
  if constexpr (VB == 2) {
    static_assert(kWaves * 64 == 256, "one quad per thread");
    vquad[tid] = make_uint2(vtab[tid & 15], vtab[tid >> 4]);
  }
  __syncthreads();  // q_lds and every staging slot have been read
  _Float16* const tab_t = reinterpret_cast<_Float16*>(&q_lds[0][0]);  // [th | tl][head][D]
  _Float16* const tab_qh = reinterpret_cast<_Float16*>(ring_mem + (0 * RING + RING - 1) * SG::BYTES);
  _Float16* const tab_ql = reinterpret_cast<_Float16*>(ring_mem + (1 * RING + RING - 1) * SG::BYTES);
#pragma unroll
  for (int x = 0; x < PER_T; ++x) {
    const int idx = tid + x * kWaves * 64;
    tab_t[idx] = tv[0][x];
    tab_t[kMaxGroup * D + idx] = tv[1][x];
    tab_qh[idx] = tv[2][x];
    tab_ql[idx] = tv[3][x];
  }
  __syncthreads();
  half2_t alpha[NS][4], beta[NS][4], gamma[NS][4];
  uint4_t bqa[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c0 = h * D + g * (D / 4) + 8 * s;
    const uint4_t th4 = *reinterpret_cast<const uint4_t*>(tab_t + c0);
    const uint4_t tl4 = *reinterpret_cast<const uint4_t*>(tab_t + kMaxGroup * D + c0);
    bqa[s] = *reinterpret_cast<const uint4_t*>((part ? tab_ql : tab_qh) + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t thw = th4[i], tlw = tl4[i];
      alpha[s][i] = __builtin_bit_cast(half2_t, thw);
      beta[s][i] = __builtin_bit_cast(half2_t, part ? thw : 0u);
      gamma[s][i] = __builtin_bit_cast(half2_t, part ? tlw : 0u);
    }
  }
  __syncthreads();  // every lane has its rows before the visits reuse the staging slots
  // ---- running state.  Scores, l_part and the accumulators are relative to m_ref (per
  // column, log2 units).  The value contraction's 16 columns are the 8 heads of two
  // modalities: accumulator A holds audio (columns 0-7) and video (8-15), accumulator B
  // text (0-7); the fp16 hi and lo parts of the probability operand enter as two
  // contractions into the same columns.  A window is therefore visited once, whatever
  // modalities it holds, and no accumulator ever leaves the registers.
  float m_ref = -INFINITY;
  float l_part = 0.0f;
  float4_t accA[NU], accB[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) accA[u] = accB[u] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t seen = 0u;  // modalities met (wave-uniform)
  // this lane's column modality in A and in B (kMaxModalities: none)
  const uint32_t modA = part ? 2u : 1u;
  const uint32_t modB = part ? static_cast<uint32_t>(kMaxModalities) : 0u;

  // ---- score contractions of the window in `slot` (modality-independent): the k_min
  // term cm (every A row is m_w, so each lane's results all equal q^ . m_w) and
  // scores^T = codes . (q^ (.) s_w), hi and lo columns still separate
  auto score_mma = [&](const uint8_t* slot, float4_t (&cs)[2], float4_t& cm) {
    cm = float4_t{0.f, 0.f, 0.f, 0.f};
    cs[0] = cs[1] = float4_t{0.f, 0.f, 0.f, 0.f};
    uint32_t kw[KW];
#pragma unroll
    for (int x = 0; x < KW / 4; ++x) {
      const uint4_t t = *reinterpret_cast<const uint4_t*>(slot + SG::OFF_K + 16 * (KW / 4) * lane + 16 * x);
      kw[4 * x] = t[0]; kw[4 * x + 1] = t[1]; kw[4 * x + 2] = t[2]; kw[4 * x + 3] = t[3];
    }
    if constexpr (KW == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(slot + SG::OFF_K + 8 * lane);
      kw[0] = t.x; kw[1] = t.y;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint4_t sv4 = *reinterpret_cast<const uint4_t*>(slot + SG::OFF_S + g * (D / 2) + 16 * s);
      const uint4_t mv4 = *reinterpret_cast<const uint4_t*>(slot + SG::OFF_M + g * (D / 2) + 16 * s);
      cm = mfma16(mv4, bqa[s], cm);
      // three passes over the four dwords (independent neighbours between dependent steps)
      half2_t sv[4], t[4];
      uint32_t bq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // copy the element out first: bit_cast of an ext-vector element subscript is
        // lowered as element 0 by this compiler
        const uint32_t svw = sv4[i];
        sv[i] = __builtin_bit_cast(half2_t, svw);
        t[i] = beta[s][i] * sv[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = __builtin_elementwise_fma(alpha[s][i], sv[i], -t[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) bq[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(gamma[s][i], sv[i], t[i]));
      const uint4_t bqv = uint4_t{bq[0], bq[1], bq[2], bq[3]};
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        uint4_t ak;
#pragma unroll
        for (int i = 0; i < 4; ++i) ak[i] = (kw[KO::word(tau, s, i)] >> KO::shift(tau, s, i)) & KO::mask(s);
        cs[tau] = mfma16(ak, bqv, cs[tau]);
      }
    }
  };

  // ---- MXFP4 key metadata: the slot's two raw records -> the fp16 k_scale and k_min
  // areas the score contractions read.  Lane l takes 2 D / 64 consecutive values of one
  // vector (l < 32: k_scale, else k_min), all in one 32-channel block, and converts them
  // with the block's scale (E2M1 times 2^e, exact in fp16 within its range).
  auto mx_expand = [&](uint8_t* slot) {
    constexpr int NPL = D / 32;  // values per lane
    const int vec = lane >> 5, p = lane & 31;
    if (NPL * p < D) {
      const uint8_t* raw = slot + SG::OFF_RAW + vec * SG::MXR;
      const float sc = mx_scale(raw[D / 2 + (NPL * p) / 32]);
      uint8_t* out = slot + (vec ? SG::OFF_M : SG::OFF_S) + 2 * NPL * p;
      if constexpr (NPL == 4) {
        const uint32_t nib = *reinterpret_cast<const uint16_t*>(raw + 2 * p);
        const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, sc, 0);
        const half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, sc, 1);
        *reinterpret_cast<uint2*>(out) = make_uint2(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1));
      } else {
        const uint32_t nib = raw[p];
        const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, sc, 0);
        *reinterpret_cast<uint32_t*>(out) = __builtin_bit_cast(uint32_t, v0);
      }
    }
  };

  // ---- the value contraction's A operands of the window in `slot` (fp16 levels, channel
  // tile u: row = channel, the lane's 8 tokens), built from the value block and the level
  // tables; the same for every accumulator.  Built right after the score contractions are
  // issued, their table reads overlap those contractions.  Dwords 2 h, 2 h + 1 of tile u
  // are the level pairs of the low and high nibble of byte 2 (u & 1) + h of word u / 2:
  // 2-bit values read both with one 8-byte load of that byte's quad.
  auto value_operands = [&](const uint8_t* slot, uint4_t (&av)[NU]) {
    uint32_t vw[VW];
#pragma unroll
    for (int x = 0; x < VW / 4; ++x) {
      const uint4_t t = *reinterpret_cast<const uint4_t*>(slot + SG::OFF_V + 16 * (VW / 4) * lane + 16 * x);
      vw[4 * x] = t[0]; vw[4 * x + 1] = t[1]; vw[4 * x + 2] = t[2]; vw[4 * x + 3] = t[3];
    }
    if constexpr (VW == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(slot + SG::OFF_V + 8 * lane);
      vw[0] = t.x; vw[1] = t.y;
    }
    if constexpr (VB == 2) {
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t byte = (vw[u / 2] >> (8 * (2 * (u & 1) + h2))) & 0xFFu;
          const uint2 e = vquad[byte];
          av[u][2 * h2] = e.x;
          av[u][2 * h2 + 1] = e.y;
        }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pp = 4 * u + i;
          av[u][i] = vtab[(vw[pp / PPW] >> (2 * VB * (pp % PPW))) & PMASK];
        }
    }
  };

  // ---- the rest of one visit of a window, given its score contractions.  Tokens count
  // when they lie inside the sequence and carry a modality tag below 3.
  auto visit = [&](const uint8_t* slot, int tokb, const float4_t (&cs)[2], const float4_t& cm,
                   const uint4_t (&av)[NU]) {
    const uint32_t tg0 = *reinterpret_cast<const uint32_t*>(slot + SG::OFF_TAG + 4 * g);
    const uint32_t tg1 = *reinterpret_cast<const uint32_t*>(slot + SG::OFF_TAG + 16 + 4 * g);
    // value scales of this lane's tokens, fp16 pairs (tokens 4g.., then 16 + 4g..)
    const uint2 sig0 = *reinterpret_cast<const uint2*>(slot + SG::OFF_SIG + 2 * (4 * g));
    const uint2 sig1 = *reinterpret_cast<const uint2*>(slot + SG::OFF_SIG + 2 * (16 + 4 * g));
    uint32_t sgw[4] = {sig0.x, sig0.y, sig1.x, sig1.y};
    // ---- the common case: one modality over a whole window inside the sequence.  Lane 0
    // holds tokens 0 .. 3 in tg0, so its low byte is token 0's tag.
    const uint32_t t00 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tg0))) & 0xFFu;
    const uint32_t rep = t00 * 0x01010101u;
    const bool full = tokb + kWindow <= len;
    const bool uniform = t00 < static_cast<uint32_t>(kMaxModalities) && full &&
                         (__builtin_amdgcn_ballot_w64(tg0 == rep) & __builtin_amdgcn_ballot_w64(tg1 == rep)) ==
                             __builtin_amdgcn_read_exec();
    // the next most common case: a window inside the sequence whose tags are all below 3
    // (several modalities, every token counts), which needs no masking
    bool clean = uniform;
    // ---- scores relative to m_ref (the first visit of a wave takes absolute scores)
    // (every column's reference is set at the first visit: one lane speaks for the wave)
    const bool fresh = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m_ref)) == __builtin_bit_cast(int, -INFINITY);
    // hi + lo column sums (lane n + 8's column into lane n's).  The empty asm keeps each sum
    // in the block of its DPP move (the move, convergent, stays put; a sum sunk into a later
    // block could not fold into it), so the pair becomes one v_add_f32_dpp.
    float aws = cm[0] + row_ror8(cm[0]);
    float hl[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) hl[tau][i] = cs[tau][i] + row_ror8(cs[tau][i]);
    asm volatile("" : "+v"(aws), "+v"(hl[0][0]), "+v"(hl[0][1]), "+v"(hl[0][2]), "+v"(hl[0][3]),
                 "+v"(hl[1][0]), "+v"(hl[1][1]), "+v"(hl[1][2]), "+v"(hl[1][3]));
    const float aw = aws * zh;
    const float base = fresh ? aw : aw - m_ref;
    float sc[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[tau][i] = fmaf(hl[tau][i], zfac, base);
    if (!uniform) {
      static_assert(kMaxModalities == 3, "tags 0, 1, 2 are the bit patterns 00, 01, 10 of a byte");
      const uint32_t three = (tg0 & (tg0 >> 1)) | (tg1 & (tg1 >> 1));  // bit 0 of a byte: both bits set
      clean = full && wave_all((((tg0 | tg1) & 0xFCFCFCFCu) | (three & 0x01010101u)) == 0u);
    }
    if (!clean) {
      // a real branch: the masking is rare, keep it off the common path
      asm volatile("" ::: "memory");
      bool any_counted = false;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const uint32_t tw = tau ? tg1 : tg0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (tokb + 16 * tau + 4 * g + i < len) && ((tw >> (8 * i)) & 0xFFu) < static_cast<uint32_t>(kMaxModalities);
          if (!ok) sc[tau][i] = -INFINITY;
          any_counted = any_counted || ok;
        }
        // tokens that do not count get p = 0 and, as their scale bits may be anything, a
        // zero scale
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sgw[2 * tau + e] &= (sc[tau][2 * e] == -INFINITY ? 0u : 0x0000FFFFu) |
                              (sc[tau][2 * e + 1] == -INFINITY ? 0u : 0xFFFF0000u);
        }
      }
      // with tags in range every window inside the sequence has a counted token; a window
      // without one (tags out of range) is skipped, which keeps the column max finite
      if (!wave_any(any_counted)) return;
    }
    // ---- probabilities and the range of p sigma.  p sigma enters the value contraction as
    // fp16 hi and lo parts; the reference moves when a lane's largest hi part passes 2^kXMax
    // (or is not finite: as fp16 bit patterns of values >= 0 order like integers), and the
    // window's probabilities are then recomputed.  The first visit sets the reference.
    float p[8];
    uint32_t bhi[4], blo[4];
    const uint32_t zero4[4] = {0u, 0u, 0u, 0u};
    auto probabilities = [&]() {
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = exp2_raw(sc[k >> 2][k & 3]);
      mix_quad(p, sgw, zero4, bhi);
    };
    // (fresh is wave-uniform, so the vote below is one comparison's lane mask)
    bool move = true;
    if (!fresh) {
      probabilities();
      const ushort2_t a = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, bhi[0]), __builtin_bit_cast(ushort2_t, bhi[1]));
      const ushort2_t b2 = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, bhi[2]), __builtin_bit_cast(ushort2_t, bhi[3]));
      const ushort2_t c2 = __builtin_elementwise_max(a, b2);
      move = wave_any(max(static_cast<uint32_t>(c2.x), static_cast<uint32_t>(c2.y)) > kHiLimitBits);
    }
    if (move) {
      // log2(p sigma) + 14 < lx for every token of the lane (uncounted tokens' scales are
      // zero); every visit has a counted token, so the column max is finite
      float lmax = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, sc[tau][i]);
      const float lx = lmax + scale_exponent_field(sgw);
      const float wmax = group_max(lx);
      const bool grow = fresh || wmax > kXMax + 14.0f;
      const float delta = grow ? wmax - (kXAfter + 14.0f) : 0.0f;
      // the first visit's accumulators are still zero (and -delta may overflow exp2)
      const float alf = fresh ? 0.0f : exp2_raw(-delta);
      if (grow) m_ref = (fresh ? 0.0f : m_ref) + delta;
      l_part *= alf;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        accA[u] *= alf;
        accB[u] *= alf;
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tau][i] -= delta;
      probabilities();
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) l_part += p[k];
    mix_quad(p, sgw, bhi, blo);
    // ---- value contractions, one channel tile at a time (operands built before the visit)
    // the operand of one accumulator keeps, in each lane, the tokens of its column's
    // modality (dword qd holds tokens 2 (qd & 1), + 1 of byte group qd >> 1)
    auto keep = [&](uint32_t mod, uint32_t (&k4)[4]) {
      if (uniform) {
        const uint32_t all = t00 == mod ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) k4[qd] = all;
      } else {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const uint32_t tw = (qd >> 1) ? tg1 : tg0;
          const uint32_t ta = (tw >> (16 * (qd & 1))) & 0xFFu, tb = (tw >> (16 * (qd & 1) + 8)) & 0xFFu;
          k4[qd] = (ta == mod ? 0x0000FFFFu : 0u) | (tb == mod ? 0xFFFF0000u : 0u);
        }
      }
    };
    auto accumulate = [&](float4_t (&A)[NU], const uint32_t (&k4)[4]) {
      const uint4_t bh = uint4_t{bhi[0] & k4[0], bhi[1] & k4[1], bhi[2] & k4[2], bhi[3] & k4[3]};
      const uint4_t bl = uint4_t{blo[0] & k4[0], blo[1] & k4[1], blo[2] & k4[2], blo[3] & k4[3]};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        A[u] = mfma16(av[u], bh, A[u]);
        A[u] = mfma16(av[u], bl, A[u]);
      }
    };
    // which accumulators the window needs (wave-uniform)
    bool needA, needB;
    if (uniform) {
      needA = t00 != 0u;
      needB = t00 == 0u;
      seen |= 1u << t00;
    } else if (clean) {
      // audio and video show as a set bit 0 or 1 in some byte, text as a byte with neither
      // (bit 0 of each byte of y: the byte is not zero)
      const uint32_t o = tg0 | tg1;
      const uint32_t y = (tg0 | (tg0 >> 1)) & (tg1 | (tg1 >> 1));
      const bool a0 = (y & 0x01010101u) != 0x01010101u;
      const bool a1 = wave_any((o & 0x01010101u) != 0u), a2 = wave_any((o & 0x02020202u) != 0u);
      needA = a1 || a2;
      needB = wave_any(a0);
      seen |= (needB ? 1u : 0u) | (a1 ? 2u : 0u) | (a2 ? 4u : 0u);
    } else {
      bool a12 = false, a0 = false, a1 = false, a2 = false;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t tgi = ((tau ? tg1 : tg0) >> (8 * i)) & 0xFFu;
          const bool ok = sc[tau][i] != -INFINITY;
          a0 = a0 || (ok && tgi == 0u);
          a1 = a1 || (ok && tgi == 1u);
          a2 = a2 || (ok && tgi == 2u);
        }
      a12 = wave_any(a1 || a2);
      needA = a12;
      needB = wave_any(a0);
      seen |= (needB ? 1u : 0u) | (wave_any(a1) ? 2u : 0u) | (wave_any(a2) ? 4u : 0u);
    }
    if (needA) {
      uint32_t kA[4];
      keep(modA, kA);
      accumulate(accA, kA);
    }
    if (needB) {
      uint32_t kB[4];
      keep(modB, kB);
      accumulate(accB, kB);
    }
  };

  // ---- the visits.  Waves of two workgroups share each SIMD, and the arbiter favours the
  // older one, which would leave the younger to finish its last windows alone at a lower
  // issue rate.  Each wave therefore lowers its priority as it progresses (3 for its first
  // quarter of visits .. 0 for its last), so a wave that falls behind a quarter gets the
  // issue slots until it catches up.
  const int q1 = nw / 4, q2 = nw / 2, q3 = (3 * nw) / 4;
  int stage = 0, next_change = q1;
  uint32_t cur = 0;  // ring offset of visit i's slot
  __builtin_amdgcn_s_setprio(3);
  // Visits 0 .. nw - RING each issue the copies of the window RING - 1 ahead (the ring
  // holds RING - 1 windows in flight, as issued before the set-up) and wait with a fixed
  // count; the last RING - 1 visits issue nothing and wait for fewer groups.
  const int nsteady = nw - (RING - 1);
  for (int i = 0; i < nw; ++i) {
    if (i == next_change) {
      do {
        ++stage;
        next_change = stage == 1 ? q2 : (stage == 2 ? q3 : nw);
      } while (next_change == i);
      if (stage == 1) __builtin_amdgcn_s_setprio(2);
      else if (stage == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if (i < nsteady) {
      issue(wbeg + i + RING - 1);
      wait_vmcnt<(RING - 1) * L>();
    } else {
      // wait for this visit's copies: later visits' copies may stay in flight
      wait_groups<L, RING - 1>(issued + max(nsteady, 0) - (i + 1));
    }
    uint8_t* slot = ring_mem + wave * RING * SG::BYTES + cur;
    cur = next_slot(cur);
    if constexpr (MX) mx_expand(slot);
    float4_t cs[2], cm;
    score_mma(slot, cs, cm);
    // (kept apart: mixed into the score section, the table reads serialize its LDS loads)
    __builtin_amdgcn_sched_barrier(0);
    uint4_t av[NU];
    value_operands(slot, av);
    visit(slot, (wbeg + i) * kWindow, cs, cm, av);
    // no LDS read crosses into the next visit (a skipped window leaves its value-table reads
    // in flight; unknown to the next visit, they made each of its LDS reads wait in turn)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  }

  __builtin_amdgcn_s_setprio(0);

  // ---- epilogue: merge the block's waves into one partial.  Copies past this wave's
  // visits (issued before its length was known) are drained first; once every wave is past
  // its visits the dynamic LDS is free, and every wave stages the accumulators of the
  // modalities it met in its own [modality][head][D] region, all read after one more
  // barrier.
  wait_vmcnt<0>();
  __shared__ float2 ml_lds[kWaves][kMaxGroup];
  __shared__ __attribute__((aligned(16))) uint32_t seen_lds[kWaves];
  const float l = group_sum(l_part);
  if (lane < kMaxGroup) ml_lds[wave][lane] = make_float2(m_ref, l);  // lane < 8: column = head
  if (lane == 0) seen_lds[wave] = seen;
  __syncthreads();
  // rows of D + 16 floats: the 32 lanes of a staging write (8 heads x 4 channel quads)
  // then cover the 64 banks twice, where unpadded rows put all 8 heads on 16 banks
  constexpr int DP = D + 16;
  constexpr int RES = kMaxModalities * kMaxGroup * DP;  // floats per wave
  {
    float* const res = reinterpret_cast<float*>(ring_mem) + wave * RES;
    // modality m lives in accumulator A (audio: half 0, video: half 1) or B (text: half 0);
    // lane (n, g) of tile u holds channels 16u + 4g .. +3 of column n
    auto stage = [&](int m, const float4_t (&X)[NU], int half) {
      if (((seen >> m) & 1u) && part == half) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *reinterpret_cast<float4_t*>(res + (m * kMaxGroup + h) * DP + 16 * u + 4 * g) = X[u];
      }
    };
    stage(0, accB, 0);
    stage(1, accA, 0);
    stage(2, accA, 1);
  }
  __syncthreads();
  const size_t pidx = static_cast<size_t>(unit) * a.splits + split;
  // every LDS read of the merge is unconditional and independent, so they are all in
  // flight together; what a wave did not stage (garbage) is dropped by a select
  const uint4 seen4 = *reinterpret_cast<const uint4*>(seen_lds);
  const uint32_t seen_v[kWaves] = {seen4.x, seen4.y, seen4.z, seen4.w};
  const uint32_t present = seen4.x | seen4.y | seen4.z | seen4.w;
  if (tid == 0) a.ws_mask[pidx] = present;
  const int e4 = 4 * tid;  // four consecutive elements of [head][D] per thread
  if (e4 < a.group * D) {
    const int hh = e4 / D, c4 = e4 % D;
    float2 mlv[kWaves];
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mlv[v] = ml_lds[v][hh];
    float4_t xs[kMaxModalities][kWaves];
#pragma unroll
    for (int m = 0; m < kMaxModalities; ++m)
#pragma unroll
      for (int v = 0; v < kWaves; ++v)
        if ((present >> m) & 1u)
          xs[m][v] = *reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(ring_mem) + v * RES +
                                                        (m * kMaxGroup + hh) * DP + c4);
    // the factors that bring each wave's sums to the block's max
    float mb = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mb = fmaxf(mb, mlv[v].y > 0.0f ? mlv[v].x : -INFINITY);
    float fac[kWaves];
#pragma unroll
    for (int v = 0; v < kWaves; ++v) fac[v] = mlv[v].y > 0.0f ? exp2f(mlv[v].x - mb) : 0.0f;
    if (c4 == 0) {
      float lsum = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) lsum += mlv[v].y > 0.0f ? fac[v] * mlv[v].y : 0.0f;
      a.ws_ml[pidx * kMaxGroup + hh] = make_float2(mb, lsum);
    }
#pragma unroll
    for (int m = 0; m < kMaxModalities; ++m) {
      if (!((present >> m) & 1u)) continue;
      float4_t sum = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float4_t t = xs[m][v] * fac[v];
        const bool on = (seen_v[v] >> m) & 1u;
        sum += float4_t{on ? t[0] : 0.f, on ? t[1] : 0.f, on ? t[2] : 0.f, on ? t[3] : 0.f};
      }
      *reinterpret_cast<float4_t*>(a.ws_acc + (pidx * kMaxModalities + m) * kMaxGroup * D + e4) = sum;
    }
  }
}

struct CombineArgs {
  const float* rotations_t;  // [3][d][d], Ut[m][k][c] = U_m[c][k]
  int hq, hkv, group, modalities, splits;
  const float2* ws_ml;
  const uint32_t* ws_mask;
  const float* ws_acc;
  float* out;
  // streamed sequences only: the recent tokens' partial, original space
  const float2* tail_ml;     // [unit][8]
  const float* tail_o;       // [unit][8][D]
};

// One block per (sequence x KV head, query head).  Loads that depend on nothing are issued
// first, in the order they are used: the first 64 splits' maxima, sums and masks, the
// first batch of split accumulators, then the thread's rotation rows.  Loads complete in
// issue order, and there are few enough of them (about 50) for the waits to name each one,
// so the merge starts as soon as its inputs are in.  Every wave derives the split weights
// itself (no barrier for them).
// (1) log-sum-exp merge of the splits' rotated-space accumulators, one (m, k) item per
// thread, into LDS; (2) out = sum_m U_m A_m, each thread four adjacent columns over one
// group of stacked (m, k) rows (one coalesced 16-byte load per row), the groups summed
// through LDS, then normalised.  For streamed sequences the recent tokens' partial (max,
// sum, value sums in the original space) joins the merge and is added after the rotation.
constexpr int kCombineThreads = 768;
constexpr int kCombineXB = 32;    // splits per batch of accumulator loads
constexpr int kMaxSplits = 1024;  // splits per (sequence, KV head)


template <int D, bool STREAM>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(CombineArgs a) {
  constexpr int J = kMaxModalities * D;       // stacked rotation rows (m, k)
  constexpr int CQ = D / 4;                   // threads per row group (4 columns each)
  constexpr int KQ = kCombineThreads / CQ;    // row groups
  constexpr int JPG = J / KQ;                 // rows per group
  static_assert(J % KQ == 0 && JPG % 4 == 0 && J <= kCombineThreads, "combine tiling");
  constexpr int PSTRIDE = kMaxModalities * kMaxGroup * D;  // floats per split
  __shared__ __attribute__((aligned(16))) float A[J];
  __shared__ __attribute__((aligned(16))) float red[KQ][D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = blockIdx.y, unit = blockIdx.x;
  if (h >= a.group) return;
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const size_t base = static_cast<size_t>(unit) * a.splits;
  const int S = a.splits;
  const int jrows = a.modalities * D;
  // merge item (m, k) = (tid / D, tid % D); rotation: columns 4 c4 .. 4 c4 + 3 over the
  // JPG rows of group kq
  const bool merger = tid < jrows;
  const int im = tid / D;
  const int c4 = tid % CQ, kq = tid / CQ;
  const int j0 = kq * JPG;

  // ---- loads that depend on nothing, in the order they are used (loads complete in issue
  // order): lane t's split t (max, sum) and modality mask (splits 64.. are read in the
  // loop), the first batch of split accumulators, then this thread's rotation rows - one
  // 16-byte load per row, coalesced across the row - so the merge and its barrier overlap
  // the rows still in flight
  float2 ml0 = make_float2(-INFINITY, 0.0f);
  uint32_t mk0 = 0u;
  if (lane < S) {
    ml0 = a.ws_ml[(base + lane) * kMaxGroup + h];
    mk0 = a.ws_mask[base + lane];
  }
  const float* src = a.ws_acc + base * PSTRIDE + (im * kMaxGroup + h) * D + (tid % D);
  float x[kCombineXB];
#pragma unroll
  for (int t = 0; t < kCombineXB; ++t) x[t] = (merger && t < S) ? src[static_cast<size_t>(t) * PSTRIDE] : 0.0f;
  // rows past the context's modalities read its spare rotation slots (copies of U_0, finite)
  // and meet zeros in A
  const float* up = a.rotations_t + static_cast<size_t>(j0) * D + 4 * c4;
  float4 u[JPG];
#pragma unroll
  for (int i = 0; i < JPG; ++i) u[i] = *reinterpret_cast<const float4*>(up + static_cast<size_t>(i) * D);
  // streamed sequences: the recent tokens' (max, sum) and, for row group 0, value sums
  float2 tml = make_float2(-INFINITY, 0.0f);
  float4 to = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (STREAM) {
    tml = a.tail_ml[static_cast<size_t>(unit) * kMaxGroup + h];
    if (kq == 0) to = *reinterpret_cast<const float4*>(a.tail_o + (static_cast<size_t>(unit) * kMaxGroup + h) * D + 4 * c4);
  }
  const float tmx = tml.y > 0.0f ? tml.x : -INFINITY;

  // ---- largest split max (every wave alike)
  float mx = ml0.y > 0.0f ? ml0.x : -INFINITY;
  for (int s = 64 + lane; s < S; s += 64) {
    const float2 ml = a.ws_ml[(base + s) * kMaxGroup + h];
    if (ml.y > 0.0f) mx = fmaxf(mx, ml.x);
  }
  mx = group_max(mx);
  mx = fmaxf(mx, lane_xor_row<3>(mx));
  mx = fmaxf(mx, lane_xor_row<2>(mx));
  mx = fmaxf(mx, lane_xor_row<1>(mx));
  mx = fmaxf(mx, lane_xor_row<0>(mx));
  mx = fmaxf(mx, tmx);

  // ---- (1) merge, 64 splits at a time: lane t holds split s0 + t's weight and mask.  A
  // split without modality m left that block unwritten: the mask selects, it never
  // multiplies.
  float acc = 0.0f, lsum = 0.0f;
  // splits s0 .. s0 + 63 with lane t's weight w and mask mk; the first kCombineXB of all were
  // loaded up front, the rest are read 8 at a time
  auto merge_rest = [&](int s0, float w, uint32_t mk, int from) {
    for (int sb = from; sb < min(S, s0 + 64); sb += 8) {
      float y[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = (merger && sb + t < S) ? src[static_cast<size_t>(sb + t) * PSTRIDE] : 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (sb + t >= S) break;
        // lane index of split sb + t within this group of 64 (sb - s0 + t < 64: wave-uniform)
        const int li = sb - s0 + t;
        const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), li));
        const uint32_t ms = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mk), li));
        if ((ms >> im) & 1u) acc = fmaf(ws, y[t], acc);
      }
    }
  };
  {
    // the first 64 splits, straight-line: a loop here would carry a wait for every load in
    // flight (the rotation rows included) into its first iteration
    float w = 0.0f;
    if (ml0.y > 0.0f) {
      w = exp2f(ml0.x - mx);
      lsum += w * ml0.y;
    }
#pragma unroll
    for (int t = 0; t < kCombineXB; ++t) {
      if (t < S) {
        const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), t));
        const uint32_t ms = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mk0), t));
        if ((ms >> im) & 1u) acc = fmaf(ws, x[t], acc);
      }
    }
    if (S > kCombineXB) merge_rest(0, w, mk0, kCombineXB);
  }
  if (S > 64) {
    for (int s0 = 64; s0 < S; s0 += 64) {
      float2 ml = make_float2(-INFINITY, 0.0f);
      uint32_t mk = 0u;
      if (s0 + lane < S) {
        ml = a.ws_ml[(base + s0 + lane) * kMaxGroup + h];
        mk = a.ws_mask[base + s0 + lane];
      }
      float w = 0.0f;
      if (ml.y > 0.0f) {
        w = exp2f(ml.x - mx);
        lsum += w * ml.y;
      }
      merge_rest(s0, w, mk, s0);
    }
  }
  // lanes l ^ 32, l ^ 16, then l ^ 8 .. l ^ 1 (register-to-register moves)
  lsum = group_sum(lsum);
  lsum += lane_xor_row<3>(lsum);
  lsum += lane_xor_row<2>(lsum);
  lsum += lane_xor_row<1>(lsum);
  lsum += lane_xor_row<0>(lsum);
  if (tid < J) A[tid] = merger ? acc : 0.0f;
  // ---- streamed sequences: probabilities of the recent tokens and their values, which
  // are in the original space (added after the inverse rotation)
  float4 ot = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (STREAM) {
    if (tml.y > 0.0f) {
      const float wt = exp2f(tml.x - mx);
      lsum += wt * tml.y;
      ot = make_float4(wt * to.x, wt * to.y, wt * to.z, wt * to.w);
    }
  }
  const float inv_l = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  __syncthreads();

  // ---- (2) rotation over this thread's row group: four columns
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < JPG; i += 4) {
    const float4 av = *reinterpret_cast<const float4*>(&A[j0 + i]);
    const float ai[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o.x = fmaf(u[i + r].x, ai[r], o.x);
      o.y = fmaf(u[i + r].y, ai[r], o.y);
      o.z = fmaf(u[i + r].z, ai[r], o.z);
      o.w = fmaf(u[i + r].w, ai[r], o.w);
    }
  }
  *reinterpret_cast<float4*>(&red[kq][4 * c4]) =
      make_float4(o.x + ot.x, o.y + ot.y, o.z + ot.z, o.w + ot.w);
  __syncthreads();
  if (tid < D) {
    float r = 0.0f;
#pragma unroll
    for (int g2 = 0; g2 < KQ; ++g2) r += red[g2][tid];
    a.out[(static_cast<size_t>(b) * a.hq + kvh * a.group + h) * D + tid] = r * inv_l;
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WorkspaceView {
  float2* ml;
  uint32_t* mask;
  float* acc;
  float2* tail_ml;  // streamed sequences: [unit][8]
  float* tail_o;    // [unit][8][d]
};

// [ml | mask | acc | tail_ml | tail_o], each 256-byte aligned
WorkspaceView carve(const void* ws, size_t units, size_t splits, int d) {
  const size_t parts = units * splits;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  WorkspaceView v;
  v.ml = reinterpret_cast<float2*>(w);
  w += align256(parts * kMaxGroup * sizeof(float2));
  v.mask = reinterpret_cast<uint32_t*>(w);
  w += align256(parts * sizeof(uint32_t));
  v.acc = reinterpret_cast<float*>(w);
  w += align256(parts * kMaxModalities * kMaxGroup * d * sizeof(float));
  v.tail_ml = reinterpret_cast<float2*>(w);
  w += align256(units * kMaxGroup * sizeof(float2));
  v.tail_o = reinterpret_cast<float*>(w);
  return v;
}

}  // namespace

constexpr int64_t kOldShareNum = 570, kOldShareDen = 1000;  // the older half's share of the windows

DecodePlan plan_decode(const Shape& sh, int batch, int64_t max_len, int requested, bool stream) {
  // A split is one workgroup of kWaves waves; each wave takes wpw consecutive windows
  // and the block merges its waves' partials before writing one.  Default: as many
  // workgroups as the kernel's resources let run at once (256 CUs x kBlocksPerCU), so no
  // workgroup waits for another to finish, with at least 8 windows per wave; streamed
  // sequences keep one of those places per (sequence, KV head) for the recent tokens.
  DecodePlan p{};
  const int64_t nwin = (max_len + kWindow - 1) / kWindow;
  const int64_t units = static_cast<int64_t>(batch) * sh.hkv;
  int64_t want;  // splits
  if (requested > 0) {
    want = requested;
  } else {
    const int64_t slots = 256 * kBlocksPerCU;
    want = slots / units - (stream ? 1 : 0);
    want = std::min<int64_t>(want, std::max<int64_t>(1, (nwin + 8 * kWaves - 1) / (8 * kWaves)));
  }
  want = std::max<int64_t>(1, std::min<int64_t>({want, std::max<int64_t>(1, nwin), static_cast<int64_t>(kMaxSplits)}));
  const int64_t wpw = std::max<int64_t>(1, (nwin + kWaves * want - 1) / (kWaves * want));
  const int64_t waves = std::max<int64_t>(1, (nwin + wpw - 1) / wpw);
  const int64_t splits = (waves + kWaves - 1) / kWaves;
  p.splits = static_cast<int>(splits);
  p.windows_per_wave = static_cast<int>(wpw);
  p.split_old = 0;
  p.wpw_young = static_cast<int>(wpw);
  // The launch is split-major: the workgroups of splits below 256 / units are dispatched
  // first, one per CU, and the SIMD arbiter favours their waves over the later ones that
  // share the CU.  With a full machine they take a larger share of the windows, so the two
  // finish together.
  const int64_t old = 256 / units;
  if (requested <= 0 && old >= 1 && old < splits && splits * units >= 2 * 256 - units) {
    const int64_t wo = std::max<int64_t>(1, (nwin * kOldShareNum + kWaves * old * kOldShareDen - 1) / (kWaves * old * kOldShareDen));
    const int64_t rest = std::max<int64_t>(0, nwin - kWaves * old * wo);
    const int64_t wy = (rest + kWaves * (splits - old) - 1) / (kWaves * (splits - old));
    p.split_old = static_cast<int>(old);
    p.windows_per_wave = static_cast<int>(wo);
    p.wpw_young = static_cast<int>(wy);
  }
  const size_t parts = static_cast<size_t>(units) * splits;
  p.workspace_bytes = align256(parts * kMaxGroup * sizeof(float2)) + align256(parts * sizeof(uint32_t)) +
                      align256(parts * kMaxModalities * kMaxGroup * sh.d * sizeof(float)) +
                      align256(static_cast<size_t>(units) * kMaxGroup * sizeof(float2)) +
                      align256(static_cast<size_t>(units) * kMaxGroup * sh.d * sizeof(float));
  return p;
}

template <int D, int KB, int VB, bool MX>
static hipError_t launch_partial_t(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                   const float* q, const int32_t* seq_lens, int batch, int64_t max_len,
                                   const uint32_t* kc, const uint16_t* km, const uint16_t* ks,
                                   const uint32_t* vc, const uint16_t* vs, const uint8_t* mod,
                                   int64_t t_cap, float scale, void* ws, const StreamTail* tail, hipStream_t st) {
  const WorkspaceView w = carve(ws, static_cast<size_t>(batch) * sh.hkv, plan.splits, sh.d);
  PartialArgs pa{q, seq_lens, kc, km, ks, vc, vs, mod, tb.signs, tb.pair_table, sh.hq, sh.hkv, sh.group,
                 sh.modalities, t_cap, max_len, scale * 1.4426950408889634f, plan.windows_per_wave, plan.splits,
                 plan.split_old, plan.wpw_young, w.ml, w.mask, w.acc, tail ? 1 : 0,
                 tail ? tail->k_ring : nullptr, tail ? tail->v_ring : nullptr, tail && tail->ring_f32 ? 1 : 0,
                 tail ? tail->ring_cap : 0, w.tail_ml, w.tail_o};
  // streamed sequences: one more workgroup per unit for the recent tokens
  const dim3 grid(static_cast<unsigned>(batch * sh.hkv), static_cast<unsigned>(plan.splits + (tail ? 1 : 0)));
  constexpr size_t dyn_bytes = Lds<D, KB, VB, MX>::DYN;
  // dynamic LDS above the 64 KB default needs the attribute, once per device (setting it
  // twice from two threads is harmless)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit == 0 || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_partial_kernel<D, KB, VB, MX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(dyn_bytes));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  decode_partial_kernel<D, KB, VB, MX><<<grid, kWaves * 64, dyn_bytes, st>>>(pa);
  return hipGetLastError();
}

hipError_t launch_decode_partial(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan, const float* q,
                                 const int32_t* seq_lens, int batch, int64_t max_len, const uint32_t* kc,
                                 const uint16_t* km, const uint16_t* ks, const uint32_t* vc, const uint16_t* vs,
                                 const uint8_t* mod, int64_t t_cap, float scale, void* ws, const StreamTail* tail,
                                 hipStream_t st) {
#define OMNIKV_DEC(D_, KB_, VB_)                                                                                  \
  if (sh.d == D_ && sh.kbits == KB_ && sh.vbits == VB_)                                                           \
    return sh.mx ? launch_partial_t<D_, KB_, VB_, true>(sh, tb, plan, q, seq_lens, batch, max_len, kc, km, ks, vc, \
                                                        vs, mod, t_cap, scale, ws, tail, st)                       \
                 : launch_partial_t<D_, KB_, VB_, false>(sh, tb, plan, q, seq_lens, batch, max_len, kc, km, ks, vc, \
                                                         vs, mod, t_cap, scale, ws, tail, st);
  OMNIKV_DEC(128, 2, 2)
  OMNIKV_DEC(128, 4, 4)
  OMNIKV_DEC(128, 2, 4)
  OMNIKV_DEC(128, 4, 2)
  OMNIKV_DEC(64, 2, 2)
  OMNIKV_DEC(64, 4, 4)
  OMNIKV_DEC(64, 2, 4)
  OMNIKV_DEC(64, 4, 2)
#undef OMNIKV_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const Shape& sh, const DeviceTables& tb, const DecodePlan& plan,
                                 const int32_t* seq_lens, int batch, const void* ws, float* out,
                                 const StreamTail* tail, hipStream_t st) {
  const WorkspaceView w = carve(ws, static_cast<size_t>(batch) * sh.hkv, plan.splits, sh.d);
  CombineArgs ca{tb.rotations_t, sh.hq, sh.hkv, sh.group, sh.modalities, plan.splits, w.ml, w.mask, w.acc, out,
                 w.tail_ml, w.tail_o};
  (void)seq_lens;
  // units fastest: workgroup i runs on XCD i % 8, and the partial's workgroups of a unit
  // (split-major grid) ran on XCD unit % 8 when the unit count is a multiple of 8, so each
  // unit's partials are read where they were written
  const dim3 grid(static_cast<unsigned>(batch * sh.hkv), static_cast<unsigned>(sh.group));
  if (sh.d == 128) {
    if (!tail) decode_combine_kernel<128, false><<<grid, kCombineThreads, 0, st>>>(ca);
    else decode_combine_kernel<128, true><<<grid, kCombineThreads, 0, st>>>(ca);
  } else {
    if (!tail) decode_combine_kernel<64, false><<<grid, kCombineThreads, 0, st>>>(ca);
    else decode_combine_kernel<64, true><<<grid, kCombineThreads, 0, st>>>(ca);
  }
  return hipGetLastError();
}

namespace {

// One block per (KV head, sequence), one thread per channel: the new token's key and
// value go to ring row lens[b] % ring_cap, its tag to modality[b][lens[b]].
template <typename T>
__global__ void stream_append_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                     const uint8_t* __restrict__ tags_new, const int32_t* __restrict__ lens,
                                     int hkv, int d, T* __restrict__ k_ring, T* __restrict__ v_ring, int ring_cap,
                                     uint8_t* __restrict__ modality, int64_t t_cap) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t len = lens[b];
  if (len < 0 || len >= t_cap || c >= d) return;  // outside the cache: nothing to write
  const size_t src = (static_cast<size_t>(b) * hkv + h) * d + c;
  const size_t dst = ((static_cast<size_t>(b) * ring_cap + len % ring_cap) * hkv + h) * d + c;
  k_ring[dst] = k_new[src];
  v_ring[dst] = v_new[src];
  if (h == 0 && c == 0) modality[static_cast<size_t>(b) * t_cap + len] = tags_new[b];
}

}  // namespace

hipError_t launch_stream_append(const Shape& sh, const void* k_new, const void* v_new, bool f32,
                                const uint8_t* tags_new, const int32_t* lens, int batch, void* k_ring,
                                void* v_ring, int ring_cap, uint8_t* modality, int64_t t_cap, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(sh.hkv), static_cast<unsigned>(batch));
  if (f32)
    stream_append_kernel<float><<<grid, sh.d, 0, st>>>(static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                                                       tags_new, lens, sh.hkv, sh.d, static_cast<float*>(k_ring),
                                                       static_cast<float*>(v_ring), ring_cap, modality, t_cap);
  else
    stream_append_kernel<uint16_t><<<grid, sh.d, 0, st>>>(
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), tags_new, lens, sh.hkv, sh.d,
        static_cast<uint16_t*>(k_ring), static_cast<uint16_t*>(v_ring), ring_cap, modality, t_cap);
  return hipGetLastError();
}

}  // namespace omnikv
