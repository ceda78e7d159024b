// qdr_kernels.hip -- gfx950 kernels of libqdr: init, quantize, dequantize, the decode step,
// window mode (token calls and the fold), chunk mode, compensator tokens.
//
// Work decomposition. One work-group of 256 threads (4 wave64) owns one (request, head)
// unit at a time. Wave w owns segment w of the tile, i.e. physical key positions
// 32w..32w+31, which all share one code width. Lane l of a wave owns value rows
// rg + 16 r (rg = l & 15, r = 0..7) at the 8 key positions 32w + 8 jg + m (jg = l >> 4,
// m = 0..7): 64 state entries per lane, held in VGPRs for the whole step.
//  - A wave-wide load of one row slot r reads 16 consecutive segment rows x 4 lanes,
//    i.e. one contiguous 64*b-byte block (512 B at 8 bits).
//  - Key-row (column) absmax stays inside a wave: in-lane over 8 rows, then across the
//    16 lanes of one DPP row. Value-row reductions (prediction, readout, value-column
//    absmax) go through LDS: 8 (wave, K or Q) partial sums or 16 (wave, jg) partial
//    maxima per row.
//  - The decode step is persistent: a grid of (CUs x resident groups) work-groups walks
//    the units, and each group moves its next unit's codes and vectors HBM -> LDS with
//    LDS-direct loads (no registers hold them) while it computes the current one, so HBM
//    reads stay in flight during the compute.
//
// Arithmetic contract (identical in every rounding to the scalar reference):
//   dequant + gate   S' = fl(code * G_ij), G_ij = fl(cf_j * rf_i) (the entry's gated step)
//   prediction       u_i = fl32(rf_i * sum_j code_ij (cf_j k_j)) in fp64
//   delta            w_i = fl(b * fl(v_i - u_i)),  S_new = fma(w_i, k_j, S')
//   readout          o_i = S_new q as rf_i sum_j code_ij (cf_j q_j) + w_i (k . q) in fp64,
//                    rounded once (compared within tolerance: S_new's entries are rounded)
//   refit            A_j = max_i |S_new_ij| (1 if 0), R_j = A_j / Qmax_j, invA = 1/A_j,
//                    y = fl(S_new * invA), c_i = max_j |y| (1 if 0), M = fl(Qmax * (1/c_i))
//   requant          field = RNE(y*M) + 2^(b-1), taken from fma(y, M, 2^23 + 2^(b-1))
//                    whose exact value lies in [2^23, 2^24) where the fp32 spacing is 1.
#include "qdr_internal.h"

namespace qdr {
namespace {

constexpr int GDN = 0;
constexpr int KDA = 1;
constexpr int RULE_STEP = 0;    // key-row ranges, then value-column scales
constexpr int RULE_KEYROW = 1;  // per-key-row INT8 baseline: c = 1
constexpr int RULE_TENSOR = 2;  // per-tensor INT8 baseline: one range per state, c = 1

// max over the 64 lanes of a wave (non-negative floats compared as unsigned ints),
// wave-uniform result
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x);

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

struct Seg {
  int bits;
  uint32_t off;  // byte offset of the segment inside the tile
};

__device__ __forceinline__ Seg seg_of(const MetaHead* mh, int w) {
  uint32_t off = 0;
  for (int s = 0; s < 4; ++s)
    if (s < w) off += 512u * mh->seg_bits[s];
  return {(int)mh->seg_bits[w], off};
}

// Raw bits of the lane's 8 codes in one segment row (row bytes = 4 * B).
struct Raw {
  uint32_t lo, hi;
};

// One 8-byte load per row for every width, so that the number and kind of memory
// instructions does not depend on the width (the lane's bytes are then selected by
// fix_raw): 8-bit: bytes [8jg, 8jg+8); 6-bit: the aligned 8 bytes holding [6jg, 6jg+6);
// 4-bit: bytes [8(jg>>1), 8(jg>>1)+8) of the 16-byte row (holds both jg pairs).
__device__ __forceinline__ uint32_t row_load_off(int B, int jg) {
  return B == 8 ? 8u * jg : (B == 6 ? (uint32_t)((jg * 6) & ~3) : 8u * (uint32_t)(jg >> 1));
}

__device__ __forceinline__ Raw load_row_any(const uint8_t* seg, int B, int row, int jg) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(seg + row * 4 * B + row_load_off(B, jg));
  Raw r;
  r.lo = p[0];
  r.hi = p[1];
  return r;
}

// select the lane's payload from the 8 loaded bytes
template <int B>
__device__ __forceinline__ Raw fix_raw(Raw x, int jg) {
  if constexpr (B == 6) {
    const uint32_t sh = (uint32_t)(jg & 1) * 16u;
    return {__builtin_amdgcn_alignbit(x.hi, x.lo, sh), (x.hi >> sh) & 0xFFFFu};
  } else if constexpr (B == 4) {
    return {(jg & 1) ? x.hi : x.lo, 0u};
  } else {
    return x;
  }
}

// field values (unsigned, offset binary) of the 8 codes as floats
template <int B>
__device__ __forceinline__ void decode_row(Raw raw, float f[8]) {
  if constexpr (B == 8) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f[m] = (float)((raw.lo >> (8 * m)) & 0xFFu);
      f[m + 4] = (float)((raw.hi >> (8 * m)) & 0xFFu);
    }
  } else if constexpr (B == 4) {
    const uint32_t ev = raw.lo & 0x0F0F0F0Fu, od = (raw.lo >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f[2 * m] = (float)((ev >> (8 * m)) & 0xFFu);
      f[2 * m + 1] = (float)((od >> (8 * m)) & 0xFFu);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 5; ++m) f[m] = (float)((raw.lo >> (6 * m)) & 0x3Fu);
    f[5] = (float)(__builtin_amdgcn_alignbit(raw.hi, raw.lo, 30) & 0x3Fu);
    f[6] = (float)((raw.hi >> 4) & 0x3Fu);
    f[7] = (float)((raw.hi >> 10) & 0x3Fu);
  }
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// t[m]: fp32 bit patterns whose low B bits hold the field and bits B..22 are zero.
// One store per row for 8 bits (8 bytes) and 4 bits (4 bytes): the 4 lanes of a row
// cover it and a wave-wide store writes 16 consecutive rows as one contiguous block.
// 6 bits (6 bytes per lane, alternating 4-byte and 2-byte alignment): dword + short.
template <int B>
__device__ __forceinline__ void store_row(uint8_t* seg, int row, int jg, const uint32_t t[8]) {
  if constexpr (B == 8) {
    // byte 0 of four words -> one word
    const uint32_t a = perm_b32(t[1], t[0], 0x0c0c0400u);  // [t0.b0, t1.b0, 0, 0]
    const uint32_t b = perm_b32(t[3], t[2], 0x0c0c0400u);
    const uint32_t c = perm_b32(t[5], t[4], 0x0c0c0400u);
    const uint32_t d = perm_b32(t[7], t[6], 0x0c0c0400u);
    *reinterpret_cast<uint2*>(seg + row * 32 + jg * 8) =
        make_uint2(perm_b32(b, a, 0x05040100u), perm_b32(d, c, 0x05040100u));
  } else if constexpr (B == 4) {
    // nibble pairs: low byte of (t[2m+1] << 4 | t[2m]) holds fields 2m, 2m+1
    const uint32_t p0 = (t[1] << 4) | t[0], p1 = (t[3] << 4) | t[2];
    const uint32_t p2 = (t[5] << 4) | t[4], p3 = (t[7] << 4) | t[6];
    *reinterpret_cast<uint32_t*>(seg + row * 16 + jg * 4) =
        perm_b32(perm_b32(p3, p2, 0x0c0c0400u), perm_b32(p1, p0, 0x0c0c0400u), 0x05040100u);
  } else {
    // 24-bit groups of 4 fields, three shift-or steps each (the empty asm keeps the
    // compiler from re-associating them into four instructions); the exponent bits of t
    // (bits 24, 25, 27, 30 of 2^23 + field) never reach bits 0..23 of a group
    auto group = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
      uint32_t x = (d << 6) | c;
      asm volatile("" : "+v"(x));
      x = (x << 6) | b;
      asm volatile("" : "+v"(x));
      return (x << 6) | a;
    };
    const uint32_t g0 = group(t[0], t[1], t[2], t[3]);
    const uint32_t g1 = group(t[4], t[5], t[6], t[7]);
    // even jg: dword at +0, short at +4; odd jg: short at +0, dword at +2 (no branch)
    uint8_t* dst = seg + row * 24 + jg * 6;
    const uint32_t par = (uint32_t)(jg & 1);
    const uint32_t dw = perm_b32(g1, g0, par ? 0x06050402u : 0x04020100u);
    const uint32_t hw = par ? g0 : (g1 >> 8);
    *reinterpret_cast<uint32_t*>(dst + 2 * par) = dw;
    *reinterpret_cast<uint16_t*>(dst + 4 - 4 * par) = (uint16_t)hw;
  }
}

__device__ __forceinline__ void load_rows(int B, const uint8_t* seg, int rg, int jg,
                                          Raw raw[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) raw[r] = load_row_any(seg, B, rg + 16 * r, jg);
}

template <int BFIX>
__device__ __forceinline__ void decode_any(int B, Raw raw, int jg, float f[8]) {
  if constexpr (BFIX != 0) {
    decode_row<BFIX>(fix_raw<BFIX>(raw, jg), f);
  } else {
    if (B == 8) decode_row<8>(raw, f);
    else if (B == 6) decode_row<6>(fix_raw<6>(raw, jg), f);
    else decode_row<4>(fix_raw<4>(raw, jg), f);
  }
}

// requantize the lane's normalised entries y (8 rows x 8 positions) and store them
template <int B>
__device__ __forceinline__ void requant_store(uint8_t* seg, int rg, int jg, const float (&y)[8][8],
                                              const float (&M)[8]) {
  const float magic = 8388608.0f + (float)(1 << (B - 1));
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t t[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) t[m] = __float_as_uint(fmaf(y[r][m], M[r], magic));
    store_row<B>(seg, rg + 16 * r, jg, t);
  }
}

template <int BFIX>
__device__ __forceinline__ void requant_any(int B, uint8_t* seg, int rg, int jg,
                                            const float (&y)[8][8], const float (&M)[8]) {
  if constexpr (BFIX != 0) {
    requant_store<BFIX>(seg, rg, jg, y, M);
  } else {
    if (B == 8) requant_store<8>(seg, rg, jg, y, M);
    else if (B == 6) requant_store<6>(seg, rg, jg, y, M);
    else requant_store<4>(seg, rg, jg, y, M);
  }
}

// max over the 16 lanes of a DPP row, for non-negative floats compared as unsigned ints
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false)); // row_ror 4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false)); // row_ror 8
  return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = row16_max_u32(x);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}

// Key-row absmax of the lane-held state s over all 128 rows of this wave's segment;
// the lanes write R (physical order) to global and 1/A to LDS for position p0 + (rg & 7).
__device__ __forceinline__ void key_row_refit(const float (&s)[8][8], int rg, int p0, int B,
                                              float* __restrict__ Rs_u, float* invA_lds) {
  uint32_t am[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    float x = fmaxf(fmaxf(fabsf(s[0][m]), fabsf(s[1][m])), fabsf(s[2][m]));
    x = fmaxf(fmaxf(x, fabsf(s[3][m])), fabsf(s[4][m]));
    x = fmaxf(fmaxf(x, fabsf(s[5][m])), fabsf(s[6][m]));
    x = fmaxf(x, fabsf(s[7][m]));
    am[m] = row16_max_u32(__float_as_uint(x));
  }
  uint32_t sel = am[0];
#pragma unroll
  for (int m = 1; m < 8; ++m) sel = ((rg & 7) == m) ? am[m] : sel;
  // lanes rg and rg + 8 hold the same value for position p0 + (rg & 7); both store it
  const float Am = __uint_as_float(sel);
  const float A = (Am == 0.0f) ? 1.0f : Am;
  Rs_u[p0 + (rg & 7)] = div_qmax(A, B);
  invA_lds[p0 + (rg & 7)] = recip_rn(A);
}

// y = s * invA in place; per-row partial value-column absmax written to cpart.
template <int STRIDE = kD>
__device__ __forceinline__ void normalise_rows(float (&s)[8][8], const float* invA_lds, int rg,
                                               int p0, int slot, float* cpart) {
  float ia[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) ia[m] = invA_lds[p0 + m];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float cm = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float y = s[r][m] * ia[m];
      s[r][m] = y;
      cm = fmaxf(cm, fabsf(y));
    }
    cpart[slot * STRIDE + rg + 16 * r] = cm;
  }
}

// ------------------------------------------------------------------------------
// init: zero state (all codes 0, R_j = 1/Qmax_j, c_i = 1)
// ------------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_init(const void* meta, int n_head,
                                                   uint32_t req_bytes, uint8_t* packed,
                                                   float* Rs, float* Cs) {
  const int u = blockIdx.x, r = u / n_head, h = u % n_head;
  const int w = wave_id(), lane = threadIdx.x & 63, rg = lane & 15, jg = lane >> 4;
  const MetaHead* mh = meta_heads(meta) + h;
  const Seg sg = seg_of(mh, w);
  uint8_t* seg = packed + (size_t)r * req_bytes + mh->tile_off + sg.off;
  float y[8][8];
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    M[rr] = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) y[rr][m] = 0.0f;
  }
  requant_any<0>(sg.bits, seg, rg, jg, y, M);
  const size_t uo = (size_t)u * kD;
  if (threadIdx.x < kD) {
    const int p = threadIdx.x;
    const int b = mh->seg_bits[p >> 5];
    Rs[uo + p] = 1.0f / (float)((1 << (b - 1)) - 1);
    Cs[uo + p] = 1.0f;
  }
}

// ------------------------------------------------------------------------------
// quantize a caller fp32 state S [unit][dv][dk] (logical order)
// ------------------------------------------------------------------------------
struct QuantLds {
  float invA[kD];
  float invc[kD];
  float cpart[16 * kD];
  uint32_t tmax[4];
};

__global__ void __launch_bounds__(kThreads) k_quantize(const void* meta, int n_head,
                                                       uint32_t req_bytes, const float* S,
                                                       uint8_t* packed, float* Rs, float* Cs,
                                                       int rule) {
  __shared__ QuantLds L;
  const int u = blockIdx.x, r = u / n_head, h = u % n_head;
  const int w = wave_id(), lane = threadIdx.x & 63, rg = lane & 15, jg = lane >> 4;
  const MetaHead* mh = meta_heads(meta) + h;
  const Seg sg = seg_of(mh, w);
  uint8_t* seg = packed + (size_t)r * req_bytes + mh->tile_off + sg.off;
  const float* Su = S + (size_t)u * kD * kD;
  const int p0 = 32 * w + 8 * jg;
  int col[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) col[m] = mh->identity ? p0 + m : (int)mh->perm[p0 + m];
  float s[8][8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr)
#pragma unroll
    for (int m = 0; m < 8; ++m) s[rr][m] = Su[(size_t)(rg + 16 * rr) * kD + col[m]];
  const size_t uo = (size_t)u * kD;
  if (rule == RULE_TENSOR) {
    // one range for the whole state
    float mx = 0.0f;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
#pragma unroll
      for (int m = 0; m < 8; ++m) mx = fmaxf(mx, fabsf(s[rr][m]));
    const uint32_t wm = wave_max_u32(__float_as_uint(mx));
    if (lane == 0) L.tmax[w] = wm;
    __syncthreads();
    const float Am = __uint_as_float(max(max(L.tmax[0], L.tmax[1]), max(L.tmax[2], L.tmax[3])));
    const float Aa = (Am == 0.0f) ? 1.0f : Am;
    if (threadIdx.x < kD) {
      const int p = threadIdx.x;
      Rs[uo + p] = div_qmax(Aa, mh->seg_bits[p >> 5]);
      L.invA[p] = recip_rn(Aa);
    }
  } else {
    key_row_refit(s, rg, p0, sg.bits, Rs + uo, L.invA);
  }
  __syncthreads();
  normalise_rows(s, L.invA, rg, p0, w * 4 + jg, L.cpart);
  __syncthreads();
  if (threadIdx.x < kD) {
    const int i = threadIdx.x;
    float cm = 0.0f;
    if (rule == RULE_STEP)
      for (int g = 0; g < 16; ++g) cm = fmaxf(cm, L.cpart[g * kD + i]);
    if (cm == 0.0f) cm = 1.0f;
    Cs[uo + i] = cm;
    L.invc[i] = recip_rn(cm);
  }
  __syncthreads();
  const float qmax = (float)((1 << (sg.bits - 1)) - 1);
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) M[rr] = qmax * L.invc[rg + 16 * rr];
  requant_any<0>(sg.bits, seg, rg, jg, s, M);
}

// ------------------------------------------------------------------------------
// dequantize: S_hat[i][j] = fl(code * fl(R_j * c_i)), logical order (the code times the
// step of its entry)
// ------------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_dequantize(const void* meta, int n_head,
                                                         uint32_t req_bytes,
                                                         const uint8_t* packed,
                                                         const float* Rs, const float* Cs,
                                                         float* S) {
  const int u = blockIdx.x, r = u / n_head, h = u % n_head;
  const int w = wave_id(), lane = threadIdx.x & 63, rg = lane & 15, jg = lane >> 4;
  const MetaHead* mh = meta_heads(meta) + h;
  const Seg sg = seg_of(mh, w);
  const uint8_t* seg = packed + (size_t)r * req_bytes + mh->tile_off + sg.off;
  Raw raw[8];
  load_rows(sg.bits, seg, rg, jg, raw);
  const size_t uo = (size_t)u * kD;
  const int p0 = 32 * w + 8 * jg;
  const float bias = (float)(1 << (sg.bits - 1));
  float R[8];
  int col[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    R[m] = Rs[uo + p0 + m];
    col[m] = mh->identity ? p0 + m : (int)mh->perm[p0 + m];
  }
  float* Su = S + (size_t)u * kD * kD;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int i = rg + 16 * rr;
    const float c = Cs[uo + i];
    float f[8];
    decode_any<0>(sg.bits, raw[rr], jg, f);
#pragma unroll
    for (int m = 0; m < 8; ++m) Su[(size_t)i * kD + col[m]] = (f[m] - bias) * (R[m] * c);
  }
}

// ------------------------------------------------------------------------------
// decode step
//
// Persistent work-groups of 4 waves walk contiguous runs of units. Wave w owns
// segment w of the current unit: its 32 key positions x 128 rows, 64 entries per lane.
// At the top of unit n every wave issues the global loads of its own share of unit
// n+1 (its tile segment and a slice of the input vectors) into registers; they land
// while unit n's prep and dot products run and are written to the (single) LDS slot
// right after the second barrier of unit n, when every wave has finished reading that
// slot and before the register peak of the update.
//
// Per unit:
//   prep  (per wave)    column/row factors, and the digit planes of its segment
//   phase 1             digit-plane sums on the matrix cores -> partials per row
//   B1 phase 2          u, w (waves 0-1) and the readout sum (waves 2-3) per row
//   B2 phase 3          the next unit's inputs to LDS; o; dequantize + gate + update;
//                       key-row absmax in the wave; normalise; per-row partial
//                       value-column maxima (at raised wave priority)
//   B3 phase 4          value-column scales (two waves, alternating per unit)
//   B4 phase 5          requantize, pack and store the segment; store the scales
// ------------------------------------------------------------------------------
constexpr int kTileMax = 16384;  // 128 x 128 codes at 8 bits

// Exact dot products on the matrix cores. The prediction needs
//   U_i = sum_j code_ij K_j,  K_j = cf_j k_j (exact in fp64),
// to fp64 accuracy. Per segment s, K is written in base-128 fixed point relative to a
// power of two above the segment's max |K|: N_j = RNE(K_j 2^(56-Es)), |N_j| < 2^55, and
//   K_j = 2^(Es-56) sum_{t<8} d_jt 128^(7-t) + e_j,  |e_j| <= 2^(Es-57),
// with 7-bit digits d (the top one signed, in [-64, 63]; the others in [0, 127]).
// Then U_i = sum_s 2^(Es-56) sum_t 128^(7-t) D_ist with D_ist = sum_j code_ij d_jt,
// exact int32 sums formed by v_mfma_i32_16x16x32_i8 (A = digit planes x positions,
// B = positions x rows). The readout uses eight digit planes of Q_j = cf_j q_j the same
// way: o_i = rf_i sum_j code_ij Q_j + w_i (k.q).
constexpr int kPlanes = 16;  // 8 planes of K, then 8 of Q

// One unit's inputs as copied from HBM (global->LDS, 16 bytes per lane).
struct VecIn {
  float k[kD], q[kD];  // logical key order
  float v[kD], R[kD];  // R: key-row scales, physical order
  float C[kD], a[kD];  // C: value-column scales; a: KDA gate, logical order
  float b, ag;               // write strength; GDN gate
  uint32_t flag[2];          // per-wave flags of the window token kernel
  uint8_t perm[kD];         // physical position -> logical key channel
};

// Partial arrays: 8 slots (wave, K or Q) or 16 slots (wave, jg) of one value per row;
// slot strides are padded so that the slots written by one instruction fall in different
// LDS banks.
constexpr int kFS = kD + 4;  // float slot stride
constexpr int kDS = kD + 2;  // double slot stride

struct StepWork {
  float cf[kD];  // column factor / s (s: the code operand's scale), physical order
  float rf[kD];  // row factor
  float kp[kD];  // k, physical order
  float w[kD];
  float invA[kD];
  float invc[kD];    // 1/c_i, or M_i = Qmax fl(1/c_i) when the width is uniform
  double osum[kD];  // rf_i-free readout sums from phase 2
  int8_t dig[4][kPlanes][4][8];  // [segment][plane][jg][operand byte]
  double scale_u[4], scale_o[4], kq[4];
  uint32_t tmax[4];  // per-wave state absmax (per-tensor rule)
  union {
    double upart[8 * kDS];   // per (wave, K or Q) combined digit-plane sums
    float cpart[16 * kFS];   // per (wave, jg) partial value-column absmax
  } part;
};

// Work order. Units are enumerated by an index k. When every head has a single code
// width, k runs width class by width class (8, 6, 4), requests in order, the class's
// heads in order; otherwise k = r * n_head + h.
struct StepArgs {
  const void* meta;
  int n_head, n_req, n_unit;
  uint32_t req_bytes;
  int uniform;
  int n_class[3];
  uint8_t* packed;
  float* Rs;
  float* Cs;
  const float* q;
  const float* k;
  const float* v;
  const float* a;
  const float* b;
  float* o;
};

// Position of a group's walk: request r, index hi among the nc heads of the class
// (or all heads), whose head numbers start at order[hoff] (uniform) or are hi itself.
struct UnitIter {
  int r, hi, nc, hoff;
};

// One unit's addressing, wave-uniform.
struct UnitInfo {
  uint32_t un;    // r * n_head + h: offset of the unit's vectors and scales / 128
  uint64_t toff;  // byte offset of the tile in the pool (pools may exceed 4 GiB)
  uint32_t sb;    // byte s = width of segment s
  uint32_t h;
};

typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;

// Scalar (constant-cache) read of dword `idx` of the metadata table.
__device__ __forceinline__ uint32_t meta_dword(const void* meta, uint32_t idx) {
  return ((cu32_ptr)meta)[idx];
}

__device__ __forceinline__ UnitInfo unit_info(const StepArgs& A, const UnitIter& it) {
  int h = it.hi;
  if (A.uniform) {
    const uint32_t pos = (uint32_t)(it.hoff + it.hi);
    const uint32_t base = (uint32_t)(sizeof(MetaHeader) + (size_t)A.n_head * sizeof(MetaHead)) / 4;
    const uint32_t d = meta_dword(A.meta, base + (pos >> 1));
    h = (int)((pos & 1) ? (d >> 16) : (d & 0xFFFFu));
  }
  const uint32_t hb = (uint32_t)(sizeof(MetaHeader) + (size_t)h * sizeof(MetaHead)) / 4;
  UnitInfo u;
  u.un = (uint32_t)(it.r * A.n_head + h);
  u.toff = (uint64_t)it.r * A.req_bytes + meta_dword(A.meta, hb);  // MetaHead::tile_off
  u.sb = meta_dword(A.meta, hb + 2);                                // MetaHead::seg_bits
  u.h = (uint32_t)h;
  return u;
}

__device__ __forceinline__ void advance(UnitIter& it) {
  if (++it.hi == it.nc) {
    it.hi = 0;
    ++it.r;
  }
}

__device__ __forceinline__ Seg seg_from(uint32_t sb, int w) {
  uint32_t off = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s)
    if (s < w) off += 512u * ((sb >> (8 * s)) & 0xFFu);
  return {(int)((sb >> (8 * w)) & 0xFFu), off};
}

// Byte of an 8-position group at which position m sits in the MFMA code operand:
// natural order for 8 bits; even positions then odd ones for 4 bits (that is how the
// nibble pairs separate into bytes); for 6 bits the first two positions of each group
// of four trade places (the order in which code_operand<6> extracts the fields).
__device__ __forceinline__ int operand_byte(int B, int m) {
  return B == 4 ? ((m & 1) ? 4 + (m >> 1) : (m >> 1)) : (B == 6 && !(m & 2) ? m ^ 1 : m);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gu32x4_ptr;
typedef const __attribute__((address_space(1))) float* gf32_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Loads straight from HBM into LDS (gfx950 LDS-direct global loads): lane l's `size`
// bytes from its own address land at lds + l * size. No register holds the data; the
// wave's vmcnt counts the load until it has landed.
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)lds, 4, 0, 0);
}

// The next unit's tile segment of wave w, 1 KB per wave-wide load, into the LDS tile
// slot. Only wave w reads segment w of the slot, so a wave may start this as soon as its
// own reads of the current segment are done -- except with mixed widths (B == 0), where
// the next unit's segments may sit at other offsets than the current unit's, which
// other waves may still be reading.
template <int B>
__device__ __forceinline__ void issue_tile(const StepArgs& A, const UnitInfo& u, int w, int lane,
                                           uint8_t* tile) {
  const Seg sg = seg_from(u.sb, w);
  const int nchunk = (B ? B : sg.bits) >> 1;  // 512 * bits bytes in 1 KB chunks
  const uint8_t* src = A.packed + u.toff + sg.off + 16 * lane;
  uint8_t* dst = tile + sg.off;
  lds_load16(src, dst);
  lds_load16(src + 1024, dst + 1024);
  if (nchunk > 2) lds_load16(src + 2048, dst + 2048);
  if (nchunk > 3) lds_load16(src + 3072, dst + 3072);
}

// The next unit's input vectors into the LDS slot (once every wave has finished reading
// the current ones). Wave w < 3 brings two consecutive VecIn arrays, lanes 0-31 the first
// and 32-63 the second, 16 bytes each:
//   wave 0: k, q      wave 1: v, R      wave 2: C, a (KDA only)
//   wave 3: the position map (lanes 0-7) where the kernel reads it -- KDA, and mixed
//           widths (B == 0), whose heads may order their channels by width (a head of a
//           single width keeps the logical order) -- and, from lane 0, b and the GDN gate.
template <int GATE, int B>
__device__ __forceinline__ void issue_vectors(const StepArgs& A, const UnitInfo& u, int w, int lane,
                                              VecIn& vin) {
  constexpr bool PERM = GATE == KDA || B == 0;
  if (w < 3) {
    const float* first = w == 0 ? A.k : (w == 1 ? A.v : A.Cs);
    const float* second = w == 0 ? A.q : (w == 1 ? A.Rs : A.a);
    const float* src = (lane < 32 ? first : second) + (size_t)u.un * kD + 4 * (lane & 31);
    if (w < 2 || GATE == KDA || lane < 32)
      lds_load16(src, reinterpret_cast<float*>(&vin) + 2 * kD * w);
  } else {
    if (PERM && lane < 8) lds_load16(meta_heads(A.meta)[u.h].perm + 16 * lane, vin.perm);
    if (lane == 0) {
      lds_load4(A.b + u.un, &vin.b);
      if (GATE == GDN) lds_load4(A.a + u.un, &vin.ag);
    }
  }
}

// max over the 32 lanes of one half of the wave
__device__ __forceinline__ int half_max_i32(int x) {
  uint32_t y = (uint32_t)(x + 4096);
  y = row16_max_u32(y);
  y = max(y, (uint32_t)__builtin_amdgcn_ds_swizzle((int)y, 0x401F));  // lane ^ 16
  return (int)y - 4096;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  // every lane's source is valid for the quad permutes and row rotations used here, so
  // no old value is needed (a plain DPP move, no zero-initialised destination)
  const int lo = __builtin_amdgcn_mov_dpp((int)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// the value of lane ^ 16 (within each half of the wave)
__device__ __forceinline__ double swap16_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_ds_swizzle((int)u, 0x401F);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(u >> 32), 0x401F);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// sum over the 32 lanes of one half of the wave; lanes 0 and 32 end with the sum taken
// in a fixed tree order
__device__ __forceinline__ double half_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);   // quad [1,0,3,2]
  x += dpp_f64<0x4E>(x);   // quad [2,3,0,1]
  x += dpp_f64<0x124>(x);  // row_ror 4
  x += dpp_f64<0x128>(x);  // row_ror 8
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_ds_swizzle((int)u, 0x401F);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(u >> 32), 0x401F);
  const double y = __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
  return x + y;
}

// Prep of wave w's segment: lanes 0-31 take K = cf k at position 32w + lane, lanes
// 32-63 take Q = cf q there (and the row factor of value row 32w + lane - 32).
template <int GATE, bool PERM>
__device__ __forceinline__ void prep(const VecIn& vin, StepWork& W, int w, int lane, int Bw) {
  const int half = lane >> 5, pl = lane & 31;
  const int p = 32 * w + pl;
  const int j = PERM ? (int)vin.perm[p] : p;
  const float kk = vin.k[j], qq = vin.q[j];
  const float cf = (GATE == KDA) ? vin.a[j] * vin.R[p] : vin.R[p];
  if (half == 0) {
    // the update's column factor cf / s (s = 1, 16, 4 at 8, 4, 6 bits: exact)
    W.cf[p] = cf * (Bw == 8 ? 1.0f : (Bw == 4 ? 0.0625f : 0.25f));
    W.kp[p] = kk;
  } else {
    W.rf[p] = (GATE == GDN) ? vin.ag * vin.C[p] : vin.C[p];
  }
  const double X = (double)cf * (double)(half ? qq : kk);
  int e = -2000;
  if (X != 0.0) (void)frexp(X, &e);
  const int E = half_max_i32(e) + 1;  // max |X| over the half < 2^(E-1)
  // N = RNE(X 2^(56-E)), |N| < 2^55: an fp64 integer, since X = cf k has at most 48
  // significant bits. Split N = h 2^28 + l (0 <= l < 2^28), then each into 7-bit digits
  // (the top one signed): plane t carries the digit of weight 128^(7-t).
  const double N = rint(ldexp(X, 56 - E));
  const double hd = floor(N * 0x1p-28);
  const int h = (int)hd, l = (int)fma(-hd, 268435456.0, N);
  int8_t* dst = &W.dig[w][8 * half][pl >> 3][operand_byte(Bw, pl & 7)];  // plane stride 32 B
  dst[0] = (int8_t)(h >> 21);
  dst[32] = (int8_t)((h >> 14) & 127);
  dst[64] = (int8_t)((h >> 7) & 127);
  dst[96] = (int8_t)(h & 127);
  dst[128] = (int8_t)(l >> 21);
  dst[160] = (int8_t)((l >> 14) & 127);
  dst[192] = (int8_t)((l >> 7) & 127);
  dst[224] = (int8_t)(l & 127);
  // k.q over all 128 channels on wave 3 only (the readout adds the four slots; the
  // others hold 0): two products per lane, then a fixed tree over the wave
  double kq = 0.0;
  if (w == 3) {
    const double pr = fma((double)vin.k[lane + 64], (double)vin.q[lane + 64],
                          (double)vin.k[lane] * (double)vin.q[lane]);
    const double hs = half_sum_f64(pr);
    const uint64_t h0 = (uint64_t)__double_as_longlong(hs);
    const uint32_t lo32 = (uint32_t)__builtin_amdgcn_readlane((int)h0, 32);
    const uint32_t hi32 = (uint32_t)__builtin_amdgcn_readlane((int)(h0 >> 32), 32);
    kq = hs + __longlong_as_double((long long)(((uint64_t)hi32 << 32) | lo32));
  }
  // the code operands are s*code with s = 1, 16, 4 for 8, 4, 6 bits
  const int ls = Bw == 8 ? 0 : (Bw == 4 ? 4 : 2);
  if (lane == 0) {
    W.scale_u[w] = ldexp(1.0, E - 56 - ls);
    W.kq[w] = kq;
  }
  if (lane == 32) W.scale_o[w] = ldexp(1.0, E - 56 - ls);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// four digit-plane sums of one row -> their base-128 combination (exact in fp64)
__device__ __forceinline__ double combine4(v4i d) {
  const int pa = d[0] * 128 + d[1];
  const int pb = d[2] * 128 + d[3];
  return fma((double)pa, 16384.0, (double)pb);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t shr16x2(uint32_t x, uint16_t a, uint16_t b) {
  const u16x2 v = __builtin_bit_cast(u16x2, x) >> (u16x2){a, b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t shl16x2(uint32_t x, uint16_t a, uint16_t b) {
  const u16x2 v = __builtin_bit_cast(u16x2, x) << (u16x2){a, b};
  return __builtin_bit_cast(uint32_t, v);
}

// Byte selectors that unpack one lane's eight 6-bit fields from the 8 bytes it loads
// (its 6 bytes start at byte 0 for even jg, byte 2 for odd jg). For a 24-bit group
// g = bytes (c0, c1, c2), U = (c0 c1 | c1 c2) as two 16-bit halves: U shifted right by
// (4, 2) puts fields 1 and 2 in bits 2-7 of bytes 0 and 2, U shifted left by (10, 0)
// puts fields 0 and 3 in bits 2-7 of bytes 1 and 3; one byte select takes those four.
struct Sel6 {
  uint32_t p0, p1;
};

__device__ __forceinline__ Sel6 sel6_for(int jg) {
  const uint32_t o = (jg & 1) ? 0x02020202u : 0u;
  return {0x02010100u + o, 0x05040403u + o};
}

// Codes of one row as signed bytes s*code in the byte order of operand_byte, where
// s = 1, 16, 4 for 8, 4, 6 bits: each field is moved to the top of its byte and its
// offset-binary bias removed. These are the MFMA B operand of the dot products and,
// converted with one signed-byte instruction, the codes of the update.
template <int B>
__device__ __forceinline__ constexpr int code_scale() {
  return B == 8 ? 1 : (B == 4 ? 16 : 4);
}

template <int B>
__device__ __forceinline__ long code_operand(Raw raw, int jg, const Sel6& sl) {
  if constexpr (B == 8) {
    const uint32_t lo = raw.lo ^ 0x80808080u, hi = raw.hi ^ 0x80808080u;
    return (long)(((uint64_t)hi << 32) | lo);
  } else if constexpr (B == 4) {
    // each nibble moved to the top of its byte, then the bias bit flipped
    const uint32_t x = (jg & 1) ? raw.hi : raw.lo;
    const uint32_t ev = ((x << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
    const uint32_t od = (x & 0xF0F0F0F0u) ^ 0x80808080u;
    return (long)(((uint64_t)od << 32) | ev);
  } else {
    const uint32_t u0 = __builtin_amdgcn_perm(raw.hi, raw.lo, sl.p0);
    const uint32_t u1 = __builtin_amdgcn_perm(raw.hi, raw.lo, sl.p1);
    // bytes [field 1, field 0, field 2, field 3] of each group, low 2 bits then cleared
    const uint32_t lo =
        (__builtin_amdgcn_perm(shl16x2(u0, 10, 0), shr16x2(u0, 4, 2), 0x07020500u) & 0xFCFCFCFCu) ^
        0x80808080u;
    const uint32_t hi =
        (__builtin_amdgcn_perm(shl16x2(u1, 10, 0), shr16x2(u1, 4, 2), 0x07020500u) & 0xFCFCFCFCu) ^
        0x80808080u;
    return (long)(((uint64_t)hi << 32) | lo);
  }
}

// One row's codes from the LDS slot (B is a compile-time width at every call): 4 bits
// reads only the lane's own word and returns it as both halves, so that the odd/even
// select of code_operand folds away.
__device__ __forceinline__ Raw lds_row(const uint8_t* seg, int B, int i, int jg) {
  if (B == 4) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(seg + i * 16 + 4 * jg);
    return {x, x};
  }
  const uint32_t* pr = reinterpret_cast<const uint32_t*>(seg + i * 4 * B + row_load_off(B, jg));
  return {pr[0], pr[1]};
}

// Phase 1 for one code width: the lane's code operands of its 8 rows (kept for the
// update) and the digit-plane sums of the prediction and the readout, combined per
// lane (4 planes of one row per 16-row block), then with the partner lane's other 4
// planes, into upart[(2 w + K/Q) * kDS + row]. The operands carry the factor
// code_scale<B>(), which the segment's sum scales remove.
template <int B>
__device__ __forceinline__ void plane_sums_raw(const StepWork& W, double* upart, const Raw (&raw)[8],
                                               int w, int rg, int jg, long (&op)[8]) {
  const long a_op = *reinterpret_cast<const long*>(&W.dig[w][rg][jg][0]);
  const v4i zero = {0, 0, 0, 0};
  const Sel6 sl = sel6_for(jg);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) op[rr] = code_operand<B>(raw[rr], jg, sl);
  // Keep the operands as built (they are reused for the update): without this the
  // compiler re-derives each field from the packed word instead of reading its byte.
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    uint32_t lo = (uint32_t)op[rr], hi = (uint32_t)((uint64_t)op[rr] >> 32);
    asm volatile("" : "+v"(lo), "+v"(hi));
    op[rr] = (long)(((uint64_t)hi << 32) | lo);
  }
  double c[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    // D[plane 4jg+t][row rg of block rr] for t = 0..3
    const v4i d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a_op, op[rr], zero, 0, 0, 0);
    const double x = combine4(d);
    // lanes jg and jg ^ 1 hold the high (planes 0-3) and low (4-7) parts of one row's K
    // (jg < 2) or Q sum; the even lane forms hi 2^28 + lo (one rounding)
    c[rr] = fma(x, 268435456.0, swap16_f64(x));
  }
  if (!(jg & 1)) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) upart[(2 * w + (jg >> 1)) * kDS + rg + 16 * rr] = c[rr];
  }
}

template <int B>
__device__ __forceinline__ void plane_sums(const StepWork& W, double* upart, const uint8_t* seg,
                                           int w, int rg, int jg, long (&op)[8]) {
  Raw raw[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) raw[rr] = lds_row(seg, B, rg + 16 * rr, jg);
  plane_sums_raw<B>(W, upart, raw, w, rg, jg, op);
}

// Phase 3 for one code width: dequantize + gate and apply the rank-one update,
//   S'_ij = fl(code_ij G_ij), G_ij = fl(cf_j rf_i),  S_new_ij = fma(w_i, k_j, S'_ij).
// The code operand holds s*code, so the column factor enters as cf / s (exact), which
// prep stored in W.cf.
template <int B>
__device__ __forceinline__ void update_phase(const StepWork& W, int rg, int p0, const long (&op)[8],
                                             float (&s)[8][8]) {
  float cfs[8], km[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    cfs[m] = W.cf[p0 + m];
    km[m] = W.kp[p0 + m];
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int i = rg + 16 * rr;
    const float rf = W.rf[i];
    const float wi = W.w[i];
    const uint32_t lo = (uint32_t)op[rr], hi = (uint32_t)((uint64_t)op[rr] >> 32);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = operand_byte(B, m);
      const uint32_t x = e < 4 ? lo : hi;
      const float code = (float)(int)(int8_t)(x >> (8 * (e & 3)));  // s * code
      s[rr][m] = fmaf(wi, km[m], code * (cfs[m] * rf));
    }
  }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t keep, uint32_t send) {
  return max(keep, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, CTRL, 0xF, 0xF, false));
}

// Key-row absmax of the lane-held state over all 128 rows of this wave's segment, as a
// reduce-scatter over the 16 lanes of a DPP row (non-negative floats compared as
// unsigned): lanes rg, rg^1 split the 8 positions 4/4, then rg, rg^2 split 2/2, then
// the 4 quads combine (rotations by 4 and 8). Lane rg ends holding positions
// 4 (rg & 1) + 2 ((rg >> 1) & 1) + {0, 1}; it finishes position
// pos = 4 (rg & 1) + 2 ((rg >> 1) & 1) + ((rg >> 2) & 1), forming R = A / Qmax when
// rg < 8 (returned, with pos, for the store) and 1/A otherwise (written to LDS).
__device__ __forceinline__ float key_row_refit_rs(const float (&s)[8][8], int rg, int p0, int B,
                                                  float* invA_lds, int& pos) {
  uint32_t x[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    float v = fmaxf(fmaxf(fabsf(s[0][m]), fabsf(s[1][m])), fabsf(s[2][m]));
    v = fmaxf(fmaxf(v, fabsf(s[3][m])), fabsf(s[4][m]));
    v = fmaxf(fmaxf(v, fabsf(s[5][m])), fabsf(s[6][m]));
    x[m] = __float_as_uint(fmaxf(v, fabsf(s[7][m])));
  }
  const bool b0 = rg & 1, b1 = (rg >> 1) & 1, b2 = (rg >> 2) & 1;
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // quad [1,0,3,2]
    y[i] = dpp_max_u32<0xB1>(b0 ? x[i + 4] : x[i], b0 ? x[i] : x[i + 4]);
  uint32_t z[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)  // quad [2,3,0,1]
    z[k] = dpp_max_u32<0x4E>(b1 ? y[k + 2] : y[k], b1 ? y[k] : y[k + 2]);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    z[k] = dpp_max_u32<0x124>(z[k], z[k]);  // row_ror 4
    z[k] = dpp_max_u32<0x128>(z[k], z[k]);  // row_ror 8
  }
  pos = 4 * (int)b0 + 2 * (int)b1 + (int)b2;
  const float Am = __uint_as_float(b2 ? z[1] : z[0]);
  const float A = (Am == 0.0f) ? 1.0f : Am;
  const bool rlane = rg < 8;
  const float r = rlane ? div_qmax(A, B) : recip_rn(A);
  if (!rlane) invA_lds[p0 + pos] = r;
  return r;
}

__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07Fu); }
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
__device__ __forceinline__ void block_sync() {
  wait_lgkm();
  __builtin_amdgcn_s_barrier();
}

// Width dispatch: B != 0 is the width of every segment; B == 0 takes the wave's own
// (wave-uniform) width at run time.
#define QDR_WIDTH_DISPATCH(B, Bw, CALL)   \
  do {                                    \
    if constexpr (B != 0) {               \
      constexpr int BB = B;               \
      CALL;                               \
    } else if (Bw == 8) {                 \
      constexpr int BB = 8;               \
      CALL;                               \
    } else if (Bw == 6) {                 \
      constexpr int BB = 6;               \
      CALL;                               \
    } else {                              \
      constexpr int BB = 4;               \
      CALL;                               \
    }                                     \
  } while (0)

// One unit. `odd` alternates the two waves that form the value-column scales. RULE is the
// scale rule of the requantization (the comparison baselines keep c = 1). `more`: there
// is a next unit `nx`, whose tile and input vectors are brought into LDS during this one.
template <int GATE, int B, int RULE>
__device__ __forceinline__ void step_unit(const StepArgs& A, uint8_t* tile, VecIn& vin, StepWork& W,
                                          const UnitInfo& cur, const UnitInfo& nx, bool more,
                                          int odd) {
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const Seg sg = seg_from(cur.sb, w);
  const int Bw = B ? B : sg.bits;
  const int p0 = 32 * w + 8 * jg;
  const size_t uo = (size_t)cur.un * kD;

  prep<GATE, GATE == KDA || B == 0>(vin, W, w, lane, Bw);
  wait_lgkm();
  __builtin_amdgcn_wave_barrier();

  // 1. code operands and digit-plane sums (matrix cores)
  long op[8];
  QDR_WIDTH_DISPATCH(B, Bw, (plane_sums<BB>(W, W.part.upart, tile + sg.off, w, rg, jg, op)));
  if (B != 0 && more) issue_tile<B>(A, nx, w, lane, tile);  // own segment read: reuse it
  block_sync();  // B1
  if (B == 0 && more) issue_tile<B>(A, nx, w, lane, tile);  // every wave is past its reads

  // 2. per row: prediction u and delta w (waves 0-1), readout sum (waves 2-3)
  {
    const int i = tid & (kD - 1);
    const double* up = &W.part.upart[i];
    if (tid < kD) {
      double U = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        U += W.scale_u[s] * up[(2 * s) * kDS];
      const float uu = (float)((double)W.rf[i] * U);
      W.w[i] = vin.b * (vin.v[i] - uu);
    } else {
      double O = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        O += W.scale_o[s] * up[(2 * s + 1) * kDS];
      W.osum[i] = O;
    }
  }
  block_sync();  // B2
  // Phase 3 is the longest stretch of VALU work and gates the group's next barrier: its
  // waves issue ahead of the other groups' waves on the SIMD (which are then mostly in
  // the latency-bound prep, matrix-core and scale phases). Measured: 4-5% per step.
  __builtin_amdgcn_s_setprio(1);

  // 3. the next unit's input vectors into LDS (every wave is past its last read of the
  //    slot); readout; dequantize + gate + update; key-row refit inside the wave; normalise
  if (more) issue_vectors<GATE, B>(A, nx, w, lane, vin);
  if (tid >= kD) {
    const int i = tid - kD;
    const double kq = ((W.kq[0] + W.kq[1]) + W.kq[2]) + W.kq[3];
    A.o[uo + i] = (float)fma((double)W.rf[i], W.osum[i], (double)W.w[i] * kq);
  }
  float s[8][8];
  QDR_WIDTH_DISPATCH(B, Bw, (update_phase<BB>(W, rg, p0, op, s)));
  int rpos;
  float Rkeep;
  if constexpr (RULE == RULE_TENSOR) {
    // one range for the whole state: wave absmax, then the four waves
    float mx = 0.0f;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
#pragma unroll
      for (int m = 0; m < 8; ++m) mx = fmaxf(mx, fabsf(s[rr][m]));
    const uint32_t wm = wave_max_u32(__float_as_uint(mx));
    if (lane == 0) W.tmax[w] = wm;
    block_sync();
    const float Am = __uint_as_float(max(max(W.tmax[0], W.tmax[1]), max(W.tmax[2], W.tmax[3])));
    const float Aa = (Am == 0.0f) ? 1.0f : Am;
    const float ia = recip_rn(Aa);
    Rkeep = div_qmax(Aa, Bw);
    rpos = rg & 7;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
#pragma unroll
      for (int m = 0; m < 8; ++m) s[rr][m] *= ia;
  } else {
    Rkeep = key_row_refit_rs(s, rg, p0, Bw, W.invA, rpos);
    wait_lgkm();
    __builtin_amdgcn_wave_barrier();
    if constexpr (RULE == RULE_STEP) {
      normalise_rows<kFS>(s, W.invA, rg, p0, w * 4 + jg, W.part.cpart);
    } else {
      float ia[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) ia[m] = W.invA[p0 + m];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
#pragma unroll
        for (int m = 0; m < 8; ++m) s[rr][m] *= ia[m];
    }
  }
  __builtin_amdgcn_s_setprio(0);
  block_sync();  // B3

  // 4. value-column scales (the baselines keep c = 1)
  float cm = 1.0f;
  if constexpr (RULE == RULE_STEP) {
    cm = 0.0f;
    if ((tid >> 7) == odd) {
      const int i = tid & (kD - 1);
#pragma unroll
      for (int g = 0; g < 16; ++g) cm = fmaxf(cm, W.part.cpart[g * kFS + i]);
      if (cm == 0.0f) cm = 1.0f;
      // one width for the whole tile: M = fl(Qmax fl(1/c_i)) once per row here
      W.invc[i] = B ? (float)((1 << (B - 1)) - 1) * recip_rn(cm) : recip_rn(cm);
    }
  }
  // the next unit's input vectors, written by every wave, must have landed before the
  // barrier that precedes their first reads
  wait_vm();
  block_sync();  // B4

  // 5. requantize and store in place; scales
  const float qmax = (float)((1 << (Bw - 1)) - 1);
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr)
    M[rr] = (RULE == RULE_STEP) ? (B ? W.invc[rg + 16 * rr] : qmax * W.invc[rg + 16 * rr]) : qmax;
  uint8_t* gseg = A.packed + cur.toff + sg.off;
  QDR_WIDTH_DISPATCH(B, Bw, (requant_store<BB>(gseg, rg, jg, s, M)));
  if (rg < 8) A.Rs[uo + p0 + rpos] = Rkeep;
  if ((tid >> 7) == odd) A.Cs[uo + (tid & (kD - 1))] = cm;
}

template <int GATE, int B, int RULE>
__device__ __forceinline__ void step_run(const StepArgs& A, uint8_t* tile, VecIn& vin, StepWork& W,
                                         UnitIter it, int count) {
  UnitInfo cur = unit_info(A, it);
  {
    const int w = wave_id(), lane = threadIdx.x & 63;
    issue_tile<B>(A, cur, w, lane, tile);
    issue_vectors<GATE, B>(A, cur, w, lane, vin);
    wait_vm();
    block_sync();
  }
  for (int n = 0; n < count; ++n) {
    advance(it);
    const bool more = n + 1 < count;
    const UnitInfo u1 = more ? unit_info(A, it) : cur;
    step_unit<GATE, B, RULE>(A, tile, vin, W, cur, u1, more, n & 1);
    cur = u1;
  }
}

template <int GATE, bool UNIFORM, int RULE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(UNIFORM ? 3 : 2)))
k_step(StepArgs A) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileMax];
  __shared__ __attribute__((aligned(16))) VecIn vin;
  __shared__ __attribute__((aligned(16))) StepWork W;
  // Work split. Uniform heads: the groups are partitioned among the width classes in
  // proportion to their units, and each group takes a contiguous run of its class
  // (one specialised loop per group). Otherwise: contiguous runs of all units.
  int k_begin, k_end, cls = 0;
  UnitIter it;
  if (UNIFORM) {
    const int G = (int)gridDim.x;
    int g0 = 0, hoff = 0;
    int gc[3], nc[3];
    for (int c = 0; c < 3; ++c) nc[c] = A.n_req * A.n_class[c];
    int left = G, nleft = A.n_unit;
    for (int c = 0; c < 3; ++c) {
      int g = nleft ? (int)(((long long)left * nc[c] + nleft / 2) / nleft) : 0;
      if (nc[c] > 0 && g < 1) g = 1;
      if (g > left) g = left;
      if (c == 2 || nc[c] == 0) g = nc[c] > 0 ? left : 0;
      gc[c] = g;
      left -= g;
      nleft -= nc[c];
    }
    while (cls < 2 && (int)blockIdx.x >= g0 + gc[cls]) {
      g0 += gc[cls];
      hoff += A.n_class[cls];
      ++cls;
    }
    const int gi = (int)blockIdx.x - g0, gn = gc[cls];
    k_begin = (int)(((long long)gi * nc[cls]) / gn);
    k_end = (int)(((long long)(gi + 1) * nc[cls]) / gn);
    it.nc = A.n_class[cls];
    it.hoff = hoff;
  } else {
    k_begin = (int)(((long long)blockIdx.x * A.n_unit) / gridDim.x);
    k_end = (int)(((long long)(blockIdx.x + 1) * A.n_unit) / gridDim.x);
    it.nc = A.n_head;
    it.hoff = 0;
  }
  if (k_begin >= k_end) return;  // uniform across the group
  it.r = k_begin / it.nc;
  it.hi = k_begin - it.r * it.nc;
  const int count = k_end - k_begin;
  if constexpr (UNIFORM) {
    if (cls == 0) step_run<GATE, 8, RULE>(A, tile, vin, W, it, count);
    else if (cls == 1) step_run<GATE, 6, RULE>(A, tile, vin, W, it, count);
    else step_run<GATE, 4, RULE>(A, tile, vin, W, it, count);
  } else {
    step_run<GATE, 0, RULE>(A, tile, vin, W, it, count);
  }
}

// ------------------------------------------------------------------------------
// window mode
//
// The packed state S0 stays fixed for W tokens. With the cumulative gate
// g_t = a_0 * ... * a_t (per key channel; GDN: the same for all channels) and the
// buffered keys decayed to time t, Kt_i(t) = k_i * a_{i+1} * ... * a_t (elementwise), the
// recurrence from S0 unrolls to
//   S_t = S0 diag(g_t) + sum_{i<=t} w_i Kt_i(t)^T,
//   w_t = b_t (v_t - S0 (g_t k_t) - sum_{i<t} w_i (Kt_i(t) . k_t)),
//   o_t = S0 (g_t q_t) + sum_{i<t} w_i (Kt_i(t) . q_t) + (k_t . q_t) w_t.
// Per token (k_window_token): S0 (g_t k_t) and S0 (g_t q_t) are exact matrix-core
// digit-plane sums (the prediction machinery of the decode step with the column factor
// cf_j = fl(g_tj R_j), row factor c_i); the buffered keys are dotted with k_t and q_t,
// eight lanes per buffered token; the row sums over buffered tokens run one thread per
// value row. The buffered keys are kept relative to a base token b: with
// h_t = a_{b+1} * ... * a_t, the buffer holds B_i = Kt_i(b) for i <= b and k_i / h_i for
// i > b, so that Kt_i(t) = B_i h_t and Kt_i(t) . k_t = B_i . (h_t k_t) -- no rewrite per
// token. When some h_t drops below 2^-80 (and at t = W-1) the base moves to t: the keys
// are decayed in place to B_i h_t = Kt_i(t) and h_t restarts at 1, which keeps every B_i
// within 2^80 of its key (gates of 0 move the base at once). At t = W-1 (k_window_fold)
// the buffered updates are folded into the state on the matrix cores (bf16 in, fp32
// accumulate, each fp32 operand split into three bf16 parts so the contraction keeps
// fp32 accuracy) and the state is refit and requantized once.
//
// Buffer of one unit (fp32): Kt[W][128] (physical key order), Wv[W][128] (value rows),
// g[128] (the cumulative gate g_t, physical order), h[128] (h_t, physical order).
// ------------------------------------------------------------------------------
constexpr int kWinMax = kWindowMax;

struct WinArgs {
  const void* meta;
  int n_head, W, t;
  uint32_t req_bytes;
  uint8_t* packed;
  float* Rs;
  float* Cs;
  uint8_t* buf;
  const float* q;
  const float* k;
  const float* v;
  const float* a;
  const float* b;
  float* o;
  // compensator tokens (m = 0: none): [n_unit][m], flat index i * 128 + j (logical j)
  int m;
  uint16_t* tok_idx;
  float* tok_val;
  int ubits;  // every head of this one width (then no metadata is read), or 0
};

__device__ __forceinline__ float* win_kt(const WinArgs& A, int u) {
  return reinterpret_cast<float*>(A.buf + (size_t)u * window_unit_bytes(A.W));
}

// WMAX: the largest window the kernel instance serves (the per-token arrays are sized to
// it; a smaller LDS footprint lets more work-groups share a CU)
// The token kernel keeps three per-position vectors in StepWork arrays it does not use
// otherwise (w: the token gate, invA: the cumulative gate, invc: q, all in physical order),
// and the alpha/beta sums over the waves in place of wave 0's partials.
template <int WMAX>
struct WinLds {
  VecIn vin;  // k, q (logical), v, R, C, a := g_t (logical), b, perm
  StepWork W;
  float ab[2][4][WMAX];  // alpha/beta partials: [which][wave][token]
  float sp[2][2][kD];  // row sums over buffered tokens: [alpha|beta][token parity][row]
  float xs[kD];        // S0 (g_t k_t) per row
  uint32_t tk_idx[64];  // the unit's compensator tokens
  float tk_val[64];
};

// Unit u's addressing from the metadata (scalar reads).
__device__ __forceinline__ UnitInfo win_unit_of(const void* meta, int n_head, uint32_t req_bytes,
                                                int u) {
  const int r = u / n_head, h = u - (u / n_head) * n_head;
  const uint32_t hb = (uint32_t)(sizeof(MetaHeader) + (size_t)h * sizeof(MetaHead)) / 4;
  UnitInfo x;
  x.un = (uint32_t)u;
  x.toff = (uint64_t)r * req_bytes + meta_dword(meta, hb);
  x.sb = meta_dword(meta, hb + 2);
  x.h = (uint32_t)h;
  return x;
}

__device__ __forceinline__ UnitInfo win_unit(const WinArgs& A, int u) {
  return win_unit_of(A.meta, A.n_head, A.req_bytes, u);
}

template <int GATE, int WMAX>
__global__ void __launch_bounds__(kThreads) k_window_token(WinArgs A) {
  __shared__ __attribute__((aligned(16))) WinLds<WMAX> L;
  float* const Lap = L.W.w;     // h_t, the buffered keys' decay since the base, physical order
  float* const Lgt = L.W.invA;  // cumulative gate, physical order
  float* const Lqp = L.W.invc;  // q, physical order
  float* const Lal = L.ab[0][0];
  float* const Lbe = L.ab[1][0];
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const int u = blockIdx.x;
  // with every head of one width the tile offset follows from the unit index and the
  // key order is the logical one: no dependent metadata load before the state's rows
  UnitInfo cur;
  if (A.ubits) {
    const int r = u / A.n_head, h = u - r * A.n_head;
    cur.un = (uint32_t)u;
    cur.toff = (uint64_t)r * A.req_bytes + (uint64_t)h * (A.req_bytes / (uint32_t)A.n_head);
    cur.sb = (uint32_t)A.ubits * 0x01010101u;
    cur.h = (uint32_t)h;
  } else {
    cur = win_unit(A, u);
  }
  const Seg sg = seg_from(cur.sb, w);
  const int Bw = sg.bits;
  const size_t uo = (size_t)u * kD;
  const int t = A.t, W = A.W;
  float* Kt = win_kt(A, u);
  float* Wv = Kt + (size_t)W * kD;
  float* gbuf = Wv + (size_t)W * kD;
  float* hbuf = gbuf + kD;
  // the fixed state's rows, straight from HBM (each is used once per token), in flight
  // while the token's vectors are staged and the digit planes formed
  Raw raw[8];
  {
    const uint8_t* seg = A.packed + cur.toff + sg.off;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) raw[rr] = load_row_any(seg, Bw, rg + 16 * rr, jg);
  }

  // 1. this token's vectors to LDS; whether the base moves to this token
  bool low = false;
  if (tid < kD) {
    const int p = tid;
    int j = p;
    if (!A.ubits) j = meta_heads(A.meta)[cur.h].perm[p];
    const float ap = (GATE == KDA) ? A.a[uo + j] : A.a[u];
    const float g = (t > 0 ? gbuf[p] : 1.0f) * ap;
    const float h = t > 0 ? hbuf[p] * ap : 1.0f;  // the base starts at token 0
    low = !(h >= 0x1p-80f);
    Lap[p] = h;
    Lgt[p] = g;
    L.vin.a[j] = g;
    L.vin.perm[p] = (uint8_t)j;
    L.vin.k[tid] = A.k[uo + tid];
    L.vin.q[tid] = A.q[uo + tid];
    L.vin.v[tid] = A.v[uo + tid];
    L.vin.R[p] = A.Rs[uo + p];
    L.vin.C[tid] = A.Cs[uo + tid];
    if (tid == 0) L.vin.b = A.b[u];
  }
  if (tid < A.m) {
    L.tk_idx[tid] = A.tok_idx[(size_t)u * A.m + tid];
    L.tk_val[tid] = A.tok_val[(size_t)u * A.m + tid];
  }
  {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(low);
    if (lane == 0 && w < 2) L.vin.flag[w] = bal != 0 ? 1u : 0u;
  }
  __syncthreads();
  if (tid < kD) Lqp[tid] = L.vin.q[L.vin.perm[tid]];
  const bool rebase = t == W - 1 || (L.vin.flag[0] | L.vin.flag[1]) != 0;

  // 2. exact S0 (g_t k_t), S0 (g_t q_t): digit planes of cf k and cf q, cf = fl(g_t R)
  prep<KDA, true>(L.vin, L.W, w, lane, Bw);
  wait_lgkm();
  __builtin_amdgcn_wave_barrier();
  long op[8];
  QDR_WIDTH_DISPATCH(0, Bw, (plane_sums_raw<BB>(L.W, L.W.part.upart, raw, w, rg, jg, op)));
  __syncthreads();
  {
    const int i = tid & (kD - 1);
    const double* up = &L.W.part.upart[i];
    if (tid < kD) {
      double U = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        U += L.W.scale_u[s] * up[(2 * s) * kDS];
      L.xs[i] = (float)((double)L.W.rf[i] * U);
    } else {
      double O = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        O += L.W.scale_o[s] * up[(2 * s + 1) * kDS];
      L.W.osum[i] = O;
    }
  }

  // 3. buffered keys: dot with h_t k_t and h_t q_t (or, when the base moves, decay by h_t
  //    in place and dot with k_t and q_t) over this wave's 32 positions. Eight lanes share
  //    a buffered token (16 bytes each: one contiguous
  //    128-byte segment per token and load), eight tokens per pass; the eight partial
  //    sums combine in a fixed butterfly order.
  {
    const int sub = lane & 7, tk = lane >> 3;
    const int pb = 32 * w + 4 * sub;
    // moving the base: the keys are decayed to Kt_i(t) in place and dotted with k_t, q_t;
    // otherwise B_i is dotted with h_t k_t, h_t q_t and stays as it is
    float apl[4], kpl[4], qpl[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      apl[m] = Lap[pb + m];
      kpl[m] = rebase ? L.W.kp[pb + m] : apl[m] * L.W.kp[pb + m];
      qpl[m] = rebase ? Lqp[pb + m] : apl[m] * Lqp[pb + m];
    }
    for (int i0 = 0; i0 < t; i0 += 8) {
      const int i = i0 + tk;
      float sa = 0.0f, sb = 0.0f;
      if (i < t) {
        u32x4* kt = reinterpret_cast<u32x4*>(Kt + (size_t)i * kD + pb);
        u32x4 x = *kt;
        if (rebase) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float e = __uint_as_float(x[m]) * apl[m];
            sa = fmaf(e, kpl[m], sa);
            sb = fmaf(e, qpl[m], sb);
            x[m] = __float_as_uint(e);
          }
          *kt = x;
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            sa = fmaf(__uint_as_float(x[m]), kpl[m], sa);
            sb = fmaf(__uint_as_float(x[m]), qpl[m], sb);
          }
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        sa += __shfl_xor(sa, o);
        sb += __shfl_xor(sb, o);
      }
      if (sub == 0 && i < t) {
        L.ab[0][w][i] = sa;
        L.ab[1][w][i] = sb;
      }
    }
  }
  __syncthreads();
  if (tid < t) {
    Lal[tid] = ((L.ab[0][0][tid] + L.ab[0][1][tid]) + L.ab[0][2][tid]) + L.ab[0][3][tid];
    Lbe[tid] = ((L.ab[1][0][tid] + L.ab[1][1][tid]) + L.ab[1][2][tid]) + L.ab[1][3][tid];
  }
  __syncthreads();

  // 4. per value row: sums over buffered tokens (token parity split over the halves;
  //    four independent partial sums per thread keep several loads in flight, combined
  //    in a fixed order)
  {
    const int row = tid & (kD - 1), par = tid >> 7;
    float sa[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int i = par;
    for (; i + 6 < t; i += 8) {
      float wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[u] = Wv[(size_t)(i + 2 * u) * kD + row];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sa[u] = fmaf(Lal[i + 2 * u], wv[u], sa[u]);
        sb[u] = fmaf(Lbe[i + 2 * u], wv[u], sb[u]);
      }
    }
    for (int u = 0; i < t; i += 2, ++u) {
      const float wi = Wv[(size_t)i * kD + row];
      sa[u] = fmaf(Lal[i], wi, sa[u]);
      sb[u] = fmaf(Lbe[i], wi, sb[u]);
    }
    L.sp[0][par][row] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    L.sp[1][par][row] = (sb[0] + sb[1]) + (sb[2] + sb[3]);
  }
  __syncthreads();

  // 5. delta, readout, append. The compensator tokens are entries of S0: token x at
  //    (i, j) adds x g_t,j k_t,j to the prediction and x g_t,j q_t,j to the readout of row i.
  if (tid < kD) {
    const int i = tid;
    float tu = 0.0f;
    double to = 0.0;
    for (int c = 0; c < A.m; ++c) {
      const uint32_t ix = L.tk_idx[c];
      if ((int)(ix >> 7) == i) {
        const int j = (int)(ix & (kD - 1));
        const float gx = L.tk_val[c] * L.vin.a[j];
        tu = fmaf(gx, L.vin.k[j], tu);
        to = fma((double)gx, (double)L.vin.q[j], to);
      }
    }
    const float pred = (L.xs[i] + tu) + (L.sp[0][0][i] + L.sp[0][1][i]);
    const float wt = L.vin.b * (L.vin.v[i] - pred);
    const double kq = ((L.W.kq[0] + L.W.kq[1]) + L.W.kq[2]) + L.W.kq[3];
    A.o[uo + i] = (float)(fma((double)L.W.rf[i], L.W.osum[i],
                              (double)(L.sp[1][0][i] + L.sp[1][1][i]) + to) + (double)wt * kq);
    Wv[(size_t)t * kD + i] = wt;
    Kt[(size_t)t * kD + i] = rebase ? L.W.kp[i] : L.W.kp[i] / Lap[i];  // B_t = k_t / h_t
    gbuf[i] = Lgt[i];
    hbuf[i] = rebase ? 1.0f : Lap[i];
  }
}

// Split an fp32 value into three bf16 parts whose sum is exact: each part is the top
// 8 significant bits of what is left (truncation: the bf16 is the upper half of the fp32
// pattern), so every subtraction is exact and the last part has at most 8 bits.
__device__ __forceinline__ __bf16 bf16_hi(float x) {
  return __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(x) >> 16));
}
__device__ __forceinline__ void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
  const float hf = __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
  const float r1 = x - hf;
  const float mf = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
  h = bf16_hi(hf);
  m = bf16_hi(mf);
  l = bf16_hi(r1 - mf);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Compensator tokens (LeapQuant abstract: the largest outliers kept as a few
// high-precision tokens that share the real tokens' update path): the m nonzero entries
// of largest |S| (equal magnitudes: smaller flat index i * 128 + j, j logical) are
// written out largest first and set to 0 before the refit. Candidates are the entries at
// or above T0, the m-th largest of the 64 lane-quad maxima (m <= 16) or of the 256
// per-thread maxima (so at least m entries reach it); up to kCandCap of them are ranked
// in LDS. More candidates (many equal magnitudes) take an exact bisection over the
// magnitude bits and then over the flat index.
constexpr int kCandCap = 1024;
constexpr int kTokMax = kCompMax;
constexpr uint32_t kTokEmpty = 0xFFFFu;
struct CompLds {
  uint2 cand[kCandCap];  // (value bits, flat index)
  uint32_t qm[kThreads];  // lane-quad (or per-thread) maxima of the magnitude bits
  uint2 tok[kTokMax];
  uint32_t n, T0;
  uint32_t part[2][4];
};

// sum over the work-group (one barrier; `r` alternates the partial slots)
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t x, uint32_t (*part)[4], int r) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) part[r & 1][threadIdx.x >> 6] = x;
  block_sync();
  return part[r & 1][0] + part[r & 1][1] + part[r & 1][2] + part[r & 1][3];
}

// Register layouts of a unit's state over the 256 threads (64 entries each): the value row
// and key position of entry x of thread (wave w, lane rg + 16 jg), and the thread and
// entry that hold (row i, position p).
// The thread's distinct positions come in NW runs of four (jbase: the first of run k,
// jword: the run of entry x).
struct ChunkLayout {  // rows 32w + 16h + rg, positions 32s + 8jg + e; x = 32h + 8s + e
  static constexpr int NW = 8;
  __device__ static int row(int x, int w, int rg) { return 32 * w + 16 * (x >> 5) + rg; }
  __device__ static int jbase(int k, int w, int jg) { return 32 * (k >> 1) + 8 * jg + 4 * (k & 1); }
  __device__ static int jword(int x) { return 2 * ((x >> 3) & 3) + ((x >> 2) & 1); }
  __device__ static int owner(int i, int p) { return (i >> 5) * 64 + (i & 15) + 16 * ((p >> 3) & 3); }
  __device__ static int slot(int i, int p) { return ((i >> 4) & 1) * 32 + (p >> 5) * 8 + (p & 7); }
};
struct FoldLayout {  // rows rg + 16rr, positions 32w + 8jg + e; x = 8rr + e
  static constexpr int NW = 2;
  __device__ static int row(int x, int w, int rg) { return rg + 16 * (x >> 3); }
  __device__ static int jbase(int k, int w, int jg) { return 32 * w + 8 * jg + 4 * k; }
  __device__ static int jword(int x) { return (x >> 2) & 1; }
  __device__ static int owner(int i, int p) { return (p >> 5) * 64 + 16 * ((p >> 3) & 3) + (i & 15); }
  __device__ static int slot(int i, int p) { return (i >> 4) * 8 + (p & 7); }
};

// The compensator tokens rejoin the register state: each token is placed by one thread
// (its owner and entry through the inverse key permutation; times gfac[p] when given,
// the gate product that the token's entry has taken since it was stored), then every
// thread adds those it owns. Their residual entries dequantize to 0. jinv must be
// visible to all threads on entry.
template <class LAYOUT>
__device__ __forceinline__ void comp_scatter(float (&S)[64], int m, const uint16_t* tok_idx,
                                             const float* tok_val, const float* gfac,
                                             uint32_t* tok_at, float* tok_v, const uint8_t* jinv) {
  const int tid = threadIdx.x;
  const int m4 = (m + 3) & ~3;
  if (tid < m4) {
    uint32_t at = 0xFFFFFFFFu;
    float val = 0.0f;
    if (tid < m) {
      const uint32_t ix = tok_idx[tid];
      if (ix < (uint32_t)(kD * kD)) {
        const int i = (int)(ix >> 7), p = jinv[ix & (kD - 1)];
        at = (uint32_t)LAYOUT::owner(i, p) << 8 | (uint32_t)LAYOUT::slot(i, p);
        val = gfac ? tok_val[tid] * gfac[p] : tok_val[tid];
      }
    }
    tok_at[tid] = at;
    tok_v[tid] = val;
  }
  block_sync();
  for (int t = 0; t < m4; t += 4) {
    const uint4 at4 = *reinterpret_cast<const uint4*>(&tok_at[t]);
    const uint32_t ats[4] = {at4.x, at4.y, at4.z, at4.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((ats[c] >> 8) == (uint32_t)tid) {
        const float val = tok_v[t + c];
        const int sl = (int)(ats[c] & 63u);
#pragma unroll
        for (int x = 0; x < 64; ++x)
          if (x == sl) S[x] += val;
      }
    }
  }
}

// Selection of the new tokens from the register state (see above); writes tok_idx /
// tok_val [m] of the unit and zeroes the selected entries. jperm must be visible to all
// threads on entry; C is scratch that no thread uses until this returns.
template <class LAYOUT>
__device__ __forceinline__ void comp_select(float (&S)[64], int m_, uint16_t* tok_idx,
                                            float* tok_val, CompLds& C, const uint8_t* jperm) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const uint32_t m = (uint32_t)m_;
  // logical key channels of the thread's positions, four per word
  uint32_t jp[LAYOUT::NW];
#pragma unroll
  for (int k = 0; k < LAYOUT::NW; ++k)
    jp[k] = *reinterpret_cast<const uint32_t*>(&jperm[LAYOUT::jbase(k, w, jg)]);
  auto key = [&](int x) { return __float_as_uint(S[x]) & 0x7FFFFFFFu; };
  auto flat = [&](int x) {
    return (uint32_t)(LAYOUT::row(x, w, rg) * kD) + ((jp[LAYOUT::jword(x)] >> (8 * (x & 3))) & 0xFFu);
  };
  uint32_t tmax = 0;
#pragma unroll
  for (int x = 0; x < 64; ++x) tmax = max(tmax, key(x));
  const bool quads = m <= 16;
  if (quads) {
    tmax = max(tmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)tmax, 0xB1, 0xF, 0xF, false));
    tmax = max(tmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)tmax, 0x4E, 0xF, 0xF, false));
    if ((lane & 3) == 0) C.qm[tid >> 2] = tmax;
  } else {
    C.qm[tid] = tmax;
  }
  if (tid == 0) {
    C.n = 0;
    C.T0 = 0;
  }
  block_sync();
  // T0: the largest maximum that at least m of the maxima reach
  if (quads) {
    if (w == 0) {
      const uint32_t x = C.qm[lane];
      uint32_t ge = 0;
#pragma unroll 16
      for (int j = 0; j < 64; ++j)
        ge += (uint32_t)((uint32_t)__builtin_amdgcn_readlane((int)x, j) >= x);
      const uint32_t t0 = wave_max_u32(ge >= m ? x : 0u);
      if (lane == 0) C.T0 = t0;
    }
  } else {
    // the m-th largest of the 256 maxima, built bit by bit from the top (magnitudes: bit
    // 31 is clear) from ballot counts; every wave finds the same value, wave 0 stores it
    const uint32_t y0 = C.qm[lane], y1 = C.qm[64 + lane], y2 = C.qm[128 + lane],
                   y3 = C.qm[192 + lane];
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      const uint32_t cnt = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(y0 >= c)) +
                           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(y1 >= c)) +
                           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(y2 >= c)) +
                           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(y3 >= c));
      if (cnt >= m) T = c;
    }
    if (tid == 0) C.T0 = T;
  }
  block_sync();
  // candidates: |S| >= T0 and nonzero (T0 raised to the smallest positive magnitude).
  // The wave counts its candidates, takes one range of slots, then writes them in order.
  const float T0f = __uint_as_float(max(C.T0, 1u));
  {
    uint32_t cnt = 0;
#pragma unroll
    for (int x = 0; x < 64; ++x)
      cnt += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(fabsf(S[x]) >= T0f));
    uint32_t base = 0;
    if (lane == 0 && cnt) base = atomicAdd(&C.n, cnt);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
    for (int x = 0; x < 64; ++x) {
      const bool c = fabsf(S[x]) >= T0f;
      const uint64_t mk = __builtin_amdgcn_ballot_w64(c);
      if (mk) {
        const uint32_t slot =
            base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
        if (c && slot < (uint32_t)kCandCap)
          C.cand[slot] = make_uint2(__float_as_uint(S[x]), flat(x));
        base += (uint32_t)__builtin_popcountll(mk);
      }
    }
  }
  block_sync();
  uint32_t n = C.n;
  if (n > (uint32_t)kCandCap) {
    // the m-th largest magnitude T (n > kCandCap >= m nonzero entries exist), then the
    // flat-index cut among the entries of magnitude T
    int r = 0;
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int x = 0; x < 64; ++x) cnt += (uint32_t)(key(x) >= c);
      if (block_sum_u32(cnt, C.part, r++) >= m) T = c;
    }
    uint32_t gt = 0;
#pragma unroll
    for (int x = 0; x < 64; ++x) gt += (uint32_t)(key(x) > T);
    const uint32_t need = m - block_sum_u32(gt, C.part, r++);
    uint32_t lo = 0, hi = kD * kD - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      uint32_t cnt = 0;
#pragma unroll
      for (int x = 0; x < 64; ++x) cnt += (uint32_t)(key(x) == T && flat(x) <= mid);
      if (block_sum_u32(cnt, C.part, r++) >= need) hi = mid;
      else lo = mid + 1;
    }
    if (tid == 0) C.n = 0;
    block_sync();
#pragma unroll
    for (int x = 0; x < 64; ++x) {
      const uint32_t kk = key(x);
      if (kk >= T && (kk > T || flat(x) <= lo)) {
        const uint32_t slot = atomicAdd(&C.n, 1u);
        C.cand[slot] = make_uint2(__float_as_uint(S[x]), flat(x));
      }
    }
    block_sync();
    n = C.n;  // == m
  }
  // rank the candidates; the first m are the tokens, in order. G threads (adjacent lanes)
  // share a candidate, each scanning every G-th entry of the list; the list is padded to a
  // multiple of 8 G with zero keys, which rank below every candidate.
  uint32_t G = 1;
  while (G < 64 && 2 * G * n <= (uint32_t)kThreads) G *= 2;
  const uint32_t nP = (n + 8 * G - 1) / (8 * G) * (8 * G);
  for (uint32_t x = n + tid; x < nP; x += kThreads) C.cand[x] = make_uint2(0u, 0xFFFFFFFFu);
  block_sync();
  const uint32_t part = (uint32_t)tid & (G - 1);
  for (uint32_t c0 = 0; c0 < n; c0 += kThreads / G) {
    const uint32_t c = c0 + (uint32_t)tid / G;
    uint2 me = make_uint2(0u, 0u);
    uint32_t rk = 0;
    if (c < n) {
      me = C.cand[c];
      const uint32_t km = me.x & 0x7FFFFFFFu;
      for (uint32_t d = part; d < nP; d += 8 * G) {
        uint2 ot[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) ot[x] = C.cand[d + x * G];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const uint32_t ko = ot[x].x & 0x7FFFFFFFu;
          rk += (uint32_t)(ko > km || (ko == km && ot[x].y < me.y));
        }
      }
    }
    for (uint32_t o = 1; o < G; o <<= 1) rk += __shfl_xor(rk, (int)o);
    if (c < n && part == 0 && rk < m) C.tok[rk] = me;
  }
  block_sync();
  const uint32_t nv = min(n, m);
  if ((uint32_t)tid < m) {
    const bool valid = (uint32_t)tid < nv;
    tok_idx[tid] = valid ? (uint16_t)C.tok[tid].y : (uint16_t)kTokEmpty;
    tok_val[tid] = valid ? __uint_as_float(C.tok[tid].x) : 0.0f;
  }
  if (nv > 0) {
    // the selected entries: above the last token's magnitude, or equal to it at a flat
    // index up to the last token's
    const uint2 last = C.tok[nv - 1];
    const uint32_t kl = last.x & 0x7FFFFFFFu;
    const float klf = __uint_as_float(kl);
#pragma unroll
    for (int x = 0; x < 64; ++x) {
      const bool c = fabsf(S[x]) >= klf;
      if (__builtin_amdgcn_ballot_w64(c)) {
        const uint32_t kk = key(x);
        if (c && (kk > kl || flat(x) <= last.y)) S[x] = 0.0f;
      }
    }
  }
  block_sync();  // the scratch is reused by the refit
}

constexpr int kFoldChunk = 32;  // buffered tokens per staged chunk (one MFMA k-step)

struct FoldLds {
  float kt[kFoldChunk][kD];  // decayed keys, physical order
  float wv[kFoldChunk][kD];  // deltas, value rows
  float invA[kD];
  float invc[kD];
  float cpart[16 * kFS];
  alignas(16) uint8_t jperm[kD];  // physical position -> logical key channel
  uint8_t jinv[kD];               // logical key channel -> physical position
  uint32_t tok_at[64];            // compensator token t: owning thread << 8 | register slot
  float tok_v[64];
};
static_assert(sizeof(CompLds) <= sizeof(FoldLds::kt), "selection scratch fits");

// Fold the window into the state and requantize: S = S0 diag(g) + sum_i w_i Kt_i^T.
// COMP: with compensator tokens (A.m > 0).
template <int GATE, bool COMP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
k_window_fold(WinArgs A) {
  __shared__ __attribute__((aligned(16))) FoldLds L;
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const int u = blockIdx.x;
  const UnitInfo cur = win_unit(A, u);
  const Seg sg = seg_from(cur.sb, w);
  const int Bw = sg.bits;
  const size_t uo = (size_t)u * kD;
  const int W = A.W;
  const float* Kt = win_kt(A, u);
  const float* Wv = Kt + (size_t)W * kD;
  const float* gbuf = Wv + (size_t)W * kD;
  const int p0 = 32 * w + 8 * jg;
  if (COMP && tid < kD) {
    const int j = meta_heads(A.meta)[cur.h].perm[tid];
    L.jperm[tid] = (uint8_t)j;
    L.jinv[j] = (uint8_t)tid;
  }

  // sum_i w_i Kt_i^T on the matrix cores. Output tile (b, rr): rows rg + 16 rr, positions
  // p0 + 4b + (0..3) of this lane; A = Kt^T (16 positions x 32 tokens), B = Wv (32 tokens
  // x 16 rows).
  f32x4 d[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) d[b][rr] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  const int mrow = lane & 15, kg = lane >> 4;
  for (int i0 = 0; i0 < W; i0 += kFoldChunk) {
    __syncthreads();
    for (int e = tid; e < kFoldChunk * kD; e += kThreads) {
      const int i = i0 + e / kD;
      const bool in = i < W;
      L.kt[e / kD][e % kD] = in ? Kt[(size_t)i * kD + e % kD] : 0.0f;
      L.wv[e / kD][e % kD] = in ? Wv[(size_t)i * kD + e % kD] : 0.0f;
    }
    __syncthreads();
    bf16x8 ah[2], am[2], al[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int pos = 32 * w + 8 * (mrow >> 2) + 4 * b + (mrow & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h, m, l;
        split3(L.kt[8 * kg + e][pos], h, m, l);
        ah[b][e] = h;
        am[b][e] = m;
        al[b][e] = l;
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      bf16x8 bh, bm, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h, m, l;
        split3(L.wv[8 * kg + e][mrow + 16 * rr], h, m, l);
        bh[e] = h;
        bm[e] = m;
        bl[e] = l;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4 x = d[b][rr];
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[b], bh, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[b], bl, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[b], bm, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[b], bh, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[b], bm, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[b], bh, x, 0, 0, 0);
        d[b][rr] = x;
      }
    }
  }
  // S = S0 diag(g) + fold: S'_ij = fl(code fl(cf_j c_i)), cf_j = fl(g_j R_j), in the
  // lane layout, plus the contraction
  float s[8][8];
  {
    const uint8_t* seg = A.packed + cur.toff + sg.off;
    Raw raw[8];
    load_rows(Bw, seg, rg, jg, raw);
    const float bias = (float)(1 << (Bw - 1));
    float cf[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) cf[m] = gbuf[p0 + m] * A.Rs[uo + p0 + m];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float c = A.Cs[uo + rg + 16 * rr];
      float f[8];
      decode_any<0>(Bw, raw[rr], jg, f);
#pragma unroll
      for (int m = 0; m < 8; ++m) s[rr][m] = (f[m] - bias) * (cf[m] * c) + d[m >> 2][rr][m & 3];
    }
  }
  // compensator tokens: the stored ones rejoin S0 (decayed by the window's gate product),
  // then the new ones are selected from S and leave it before the refit
  if (COMP) {
    float(&sf)[64] = *reinterpret_cast<float(*)[64]>(&s[0][0]);
    uint16_t* ti = A.tok_idx + (size_t)u * A.m;
    float* tv = A.tok_val + (size_t)u * A.m;
    comp_scatter<FoldLayout>(sf, A.m, ti, tv, gbuf, L.tok_at, L.tok_v, L.jinv);
    comp_select<FoldLayout>(sf, A.m, ti, tv, *reinterpret_cast<CompLds*>(&L.kt[0][0]), L.jperm);
  }

  // refit + requantize (the decode step's rule)
  int rpos;
  const float Rkeep = key_row_refit_rs(s, rg, p0, Bw, L.invA, rpos);
  wait_lgkm();
  __builtin_amdgcn_wave_barrier();
  normalise_rows<kFS>(s, L.invA, rg, p0, w * 4 + jg, L.cpart);
  __syncthreads();
  float cm = 0.0f;
  if (tid < kD) {
#pragma unroll
    for (int g = 0; g < 16; ++g) cm = fmaxf(cm, L.cpart[g * kFS + tid]);
    if (cm == 0.0f) cm = 1.0f;
    L.invc[tid] = recip_rn(cm);
  }
  __syncthreads();
  const float qmax = (float)((1 << (Bw - 1)) - 1);
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) M[rr] = qmax * L.invc[rg + 16 * rr];
  uint8_t* gseg = A.packed + cur.toff + sg.off;
  QDR_WIDTH_DISPATCH(0, Bw, (requant_store<BB>(gseg, rg, jg, s, M)));
  if (rg < 8) A.Rs[uo + p0 + rpos] = Rkeep;
  if (tid < kD) A.Cs[uo + tid] = cm;
}

// ------------------------------------------------------------------------------
// chunk mode: T known tokens of every unit in one call
//
// The state is dequantized once into fp32 registers and carried through the tokens in
// sub-blocks of kCB. For a sub-block that starts after token r, with the state S_r at
// its start and the gate products gam_t = a_{r+1} ... a_t (per key channel),
//   delta_t = b_t (v_t - S_r (gam_t k_t) - sum_{i<t} A_ti delta_i),
//   o_t     = S_r (gam_t q_t) + sum_{i<=t} B_ti delta_i,
//   A_ti = sum_j k_ij k_tj a_{i+1,j} ... a_{t,j}   (i < t),  B_ti: the same with q_t,
//   S_end = S_r diag(gam_end) + sum_t delta_t (k_t a_{t+1} ... a_end)^T.
// With x_t = b_t (v_t - S_r (gam_t k_t)) and L = diag(b) A: (I + L) delta = x (forward
// substitution) and o = S_r (gam q) + B delta.
// The Grams are (k gam)(k / gam)^T and (q gam)(k / gam)^T on the matrix cores while
// every gam_end >= 2^-60 (then k / gam stays far inside the fp32 range); a sub-block
// with a smaller gate product takes them from running products of the gates read from
// memory instead (exact for any gates in [0, 1]). S_r (gam k), S_r (gam q), the Grams
// and the state update run on the matrix cores with each fp32 operand split into three
// bf16 parts (six partial products, fp32 accumulation). The state is refit and
// requantized once, after the last token (the scale rule of the decode step).
//
// Layout: wave w holds value rows 32w + 16h + rg (h = 0, 1) at key positions
// 32s + 8jg + e (segment s = 0..3, e = 0..7). A sub-block has two work-group barriers:
// one between the two halves of the gate products, one after the shared operands are in
// LDS; everything after that (Grams, products, solve, readout, update) is private to
// the wave, which owns its rows.
// ------------------------------------------------------------------------------
constexpr int kCB = 16;       // tokens per sub-block
constexpr int kRP = kD + 8;   // bf16 pitch of [token][position] operand rows
constexpr int kTP = kCB + 8;  // bf16 pitch of [position][token] operand rows (16-B aligned)

struct ChunkArgs {
  const void* meta;
  int n_head, n_unit, T;
  uint32_t req_bytes;
  uint8_t* packed;
  float* Rs;
  float* Cs;
  const float* q;  // [T][n_unit][128]
  const float* k;
  const float* v;
  const float* a;  // GDN [T][n_unit]; KDA [T][n_unit][128]
  const float* b;  // [T][n_unit]
  float* o;        // [T][n_unit][128]
  // compensator tokens (m = 0: none): [n_unit][m], flat index i * 128 + j (logical j)
  int m;
  uint16_t* tok_idx;
  float* tok_val;
  const float* S_in;  // when set: the fp32 state [n_unit][128][128] (logical), T = 0
  int ubits;          // every head of this one width (then no metadata is read), or 0
};

struct ChunkLds {
  __bf16 kpl[3][kCB][kRP];  // k_t gam_t in three bf16 parts, physical order
  __bf16 qpl[3][kCB][kRP];  // q_t gam_t
  __bf16 kmi[3][kCB][kRP];  // k_t / gam_t
  __bf16 ktl[3][kD][kTP];   // k_t a_{t+1} ... a_end, [position][token]
  float gp[4][2][kCB][kCB]; // Gram partials over each wave's segment, [t][i]
  float ex[2][kD];          // gate products over the two token halves
  float gend[kD];
  float bb[kCB];
  alignas(16) uint8_t jperm[kD];  // physical position -> logical key channel
  uint8_t jinv[kD];   // logical key channel -> physical position
  uint32_t tok_at[64];  // compensator token t: owning thread << 8 | register slot
  float tok_v[64];
};
// After the third barrier of a sub-block the operand arrays are dead; each wave then
// keeps its private arrays there.
struct ChunkPriv {
  float g[2][kCB][kCB];  // -L = -diag(b) A and B, [t][i]
};
struct ChunkX {
  float x[kCB][32];  // x_t, then delta_t, of the wave's 32 rows
};
static_assert(4 * sizeof(ChunkPriv) <= sizeof(ChunkLds::kpl), "private Grams fit");
static_assert(4 * sizeof(ChunkX) <= sizeof(ChunkLds::kmi), "private deltas fit");
static_assert(sizeof(CompLds) <= sizeof(ChunkLds::qpl), "selection scratch fits");

// One thread's share of a sub-block's inputs, loaded one sub-block ahead: tokens
// 8 (tid >> 7) + n at key position tid & 127 (k, q, a) and the value entries of its
// lane's readout slots (v).
struct ChunkPf {
  float k[8], q[8], a[8], v[8];
  float b;
};

// c += A B with A = ah + am + al and B = bh + bm + bl (bf16 parts of fp32 operands):
// the six products down to 2^-16 relative, smallest first.
__device__ __forceinline__ f32x4 mfma6_k32(bf16x8 ah, bf16x8 am, bf16x8 al, bf16x8 bh, bf16x8 bm,
                                          bf16x8 bl, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bm, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bm, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}

// requantize and store one row's 8 normalised entries y (scale M = Qmax / c_i)
template <int B>
__device__ __forceinline__ void requant_row(uint8_t* seg, int row, int jg, const float (&y)[8],
                                            float M) {
  const float magic = 8388608.0f + (float)(1 << (B - 1));
  uint32_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = __float_as_uint(fmaf(y[e], M, magic));
  store_row<B>(seg, row, jg, t);
}

__device__ __forceinline__ void wave_sync_lds() {
  wait_lgkm();
  __builtin_amdgcn_wave_barrier();
}

template <int GATE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) k_chunk(ChunkArgs A) {
  __shared__ __attribute__((aligned(16))) ChunkLds L;
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const int u = blockIdx.x;
  // With every head of one width the tile offset follows from the unit index and the
  // key order is the logical one, so the unit starts without a dependent metadata load.
  UnitInfo cur;
  const MetaHead* mh = nullptr;
  if (A.ubits) {
    const int r = u / A.n_head, h = u - r * A.n_head;
    cur.un = (uint32_t)u;
    cur.toff = (uint64_t)r * A.req_bytes + (uint64_t)h * (A.req_bytes / (uint32_t)A.n_head);
    cur.sb = (uint32_t)A.ubits * 0x01010101u;
    cur.h = (uint32_t)h;
  } else {
    cur = win_unit_of(A.meta, A.n_head, A.req_bytes, u);
    mh = meta_heads(A.meta) + cur.h;
  }
  const bool ident = A.ubits || mh->identity;
  const size_t uo = (size_t)u * kD;
  const size_t ts = (size_t)A.n_unit * kD;  // token stride of q, k, v, o (and KDA a)
  const int T = A.T;

  if (tid < kD) {
    const int j = ident ? tid : (int)mh->perm[tid];
    L.jperm[tid] = (uint8_t)j;
    L.jinv[j] = (uint8_t)tid;
  }
  const int pl = tid & (kD - 1), half = tid >> 7;
  const int jl = ident ? pl : (int)mh->perm[pl];
  // indices are clamped into range; tokens past T read as k = q = v = 0, a = 1, b = 0.
  // A sub-block with all its tokens in range forms each lane's first offset once and steps
  // it by the token stride.
  auto issue = [&](int t0, ChunkPf& f) {
    if (t0 + kCB <= T) {
      const size_t kq0 = (size_t)(t0 + 8 * half) * ts + uo + jl;
      const size_t a0 = (size_t)(t0 + 8 * half) * (size_t)A.n_unit + u;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const size_t base = kq0 + (size_t)n * ts;
        f.k[n] = A.k[base];
        f.q[n] = A.q[base];
        f.a[n] = (GATE == KDA) ? A.a[base] : A.a[a0 + (size_t)n * A.n_unit];
      }
      const size_t v0 = (size_t)(t0 + 4 * jg) * ts + uo + 32 * w + rg;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) f.v[4 * h + r] = A.v[v0 + (size_t)r * ts + 16 * h];
      f.b = A.b[(size_t)(t0 + (tid & (kCB - 1))) * A.n_unit + u];
      return;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int tt = t0 + 8 * half + n;
      const bool in = tt < T;
      const size_t ti = (size_t)(in ? tt : T - 1);
      const size_t base = ti * ts + uo;
      const float kk = A.k[base + jl], qq = A.q[base + jl];
      const float aa = (GATE == KDA) ? A.a[base + jl] : A.a[ti * A.n_unit + u];
      f.k[n] = in ? kk : 0.0f;
      f.q[n] = in ? qq : 0.0f;
      f.a[n] = in ? aa : 1.0f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + 4 * jg + r;
        const bool in = tt < T;
        const float vv = A.v[(size_t)(in ? tt : T - 1) * ts + uo + 32 * w + 16 * h + rg];
        f.v[4 * h + r] = in ? vv : 0.0f;
      }
    const int tb = t0 + (tid & (kCB - 1));
    const float bv = A.b[(size_t)(tb < T ? tb : T - 1) * A.n_unit + u];
    f.b = tb < T ? bv : 0.0f;
  };
  // the first sub-block's inputs are requested before the state is read and
  // dequantized, so that both loads are in flight together
  ChunkPf pf;
  if (T > 0) issue(0, pf);
  float S[2][4][8];
  if (A.S_in) {
    // a given fp32 state (logical key order), gathered into the register layout
    const float* Su = A.S_in + (size_t)u * kD * kD;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = 32 * s + 8 * jg + e;
        const int j = ident ? p : (int)mh->perm[p];
#pragma unroll
        for (int h = 0; h < 2; ++h) S[h][s][e] = Su[(32 * w + 16 * h + rg) * kD + j];
      }
  } else {
  // dequantize: S_ij = fl(code fl(R_j c_i)) (the decode step's readback)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const Seg sg = seg_from(cur.sb, s);
    const uint8_t* seg = A.packed + cur.toff + sg.off;
    const float bias = (float)(1 << (sg.bits - 1));
    float R[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) R[e] = A.Rs[uo + 32 * s + 8 * jg + e];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * w + 16 * h + rg;
      float f[8];
      decode_any<0>(sg.bits, load_row_any(seg, sg.bits, row, jg), jg, f);
      const float c = A.Cs[uo + row];
#pragma unroll
      for (int e = 0; e < 8; ++e) S[h][s][e] = (f[e] - bias) * (R[e] * c);
    }
  }
  // the compensator tokens rejoin the state
  if (A.m > 0) {
    block_sync();  // jinv
    comp_scatter<ChunkLayout>(*reinterpret_cast<float(*)[64]>(&S[0][0][0]), A.m,
                              A.tok_idx + (size_t)u * A.m, A.tok_val + (size_t)u * A.m, nullptr,
                              L.tok_at, L.tok_v, L.jinv);
  }
  }

  for (int t0 = 0; t0 < T; t0 += kCB) {
    // A1. gate products over this thread's 8 tokens; the two halves exchange totals
    float gl[8], sl[8];
    {
      float g = 1.0f;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        g *= pf.a[n];
        gl[n] = g;
      }
      float sf = 1.0f;
#pragma unroll
      for (int n = 7; n >= 0; --n) {
        sl[n] = sf;
        sf *= pf.a[n];
      }
      L.ex[half][pl] = g;
    }
    block_sync();

    // A2. shared operands: k gam, q gam, k / gam ([token][position]) and k decayed to
    //     the sub-block end ([position][token]), each as three bf16 parts
    {
      const float G0 = L.ex[0][pl], H1 = L.ex[1][pl];
      if (half == 0) L.gend[pl] = G0 * H1;
      __bf16 kt3[3][8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int t = 8 * half + n;
        const float gam = half ? G0 * gl[n] : gl[n];
        const float sig = half ? sl[n] : sl[n] * H1;
        __bf16 x0, x1, x2;
        split3(pf.k[n] * gam, x0, x1, x2);
        L.kpl[0][t][pl] = x0;
        L.kpl[1][t][pl] = x1;
        L.kpl[2][t][pl] = x2;
        split3(pf.q[n] * gam, x0, x1, x2);
        L.qpl[0][t][pl] = x0;
        L.qpl[1][t][pl] = x1;
        L.qpl[2][t][pl] = x2;
        split3(pf.k[n] * __builtin_amdgcn_rcpf(gam), x0, x1, x2);
        L.kmi[0][t][pl] = x0;
        L.kmi[1][t][pl] = x1;
        L.kmi[2][t][pl] = x2;
        split3(pf.k[n] * sig, kt3[0][n], kt3[1][n], kt3[2][n]);
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        bf16x8 x;
#pragma unroll
        for (int n = 0; n < 8; ++n) x[n] = kt3[c][n];
        *reinterpret_cast<bf16x8*>(&L.ktl[c][pl][8 * half]) = x;
      }
      if (tid < kCB) L.bb[tid] = pf.b;
    }
    float vcur[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) vcur[n] = pf.v[n];
    block_sync();

    // B1. per wave: S_r (gam k), S_r (gam q) and the Gram partials over the wave's own
    //     segment on the matrix cores
    bool safe;
    {
      const float g0 = L.gend[lane], g1 = L.gend[64 + lane];
      safe = __builtin_amdgcn_ballot_w64(!(g0 >= 0x1p-60f && g1 >= 0x1p-60f)) == 0;
    }
    f32x4 DA = {0.0f, 0.0f, 0.0f, 0.0f}, DB = DA, P[2] = {DA, DA}, Q[2] = {DA, DA};
    const int m = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pb0 = 32 * s + 8 * jg;
      bf16x8 kh = *reinterpret_cast<const bf16x8*>(&L.kpl[0][m][pb0]);
      bf16x8 km = *reinterpret_cast<const bf16x8*>(&L.kpl[1][m][pb0]);
      bf16x8 kl = *reinterpret_cast<const bf16x8*>(&L.kpl[2][m][pb0]);
      bf16x8 qh = *reinterpret_cast<const bf16x8*>(&L.qpl[0][m][pb0]);
      bf16x8 qm = *reinterpret_cast<const bf16x8*>(&L.qpl[1][m][pb0]);
      bf16x8 ql = *reinterpret_cast<const bf16x8*>(&L.qpl[2][m][pb0]);
      if (s == w && safe) {
        const bf16x8 ih = *reinterpret_cast<const bf16x8*>(&L.kmi[0][m][pb0]);
        const bf16x8 im = *reinterpret_cast<const bf16x8*>(&L.kmi[1][m][pb0]);
        const bf16x8 il = *reinterpret_cast<const bf16x8*>(&L.kmi[2][m][pb0]);
        DA = mfma6_k32(kh, km, kl, ih, im, il, DA);
        DB = mfma6_k32(qh, qm, ql, ih, im, il, DB);
      }
      bf16x8 bh[2], bm[2], bl[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 x0, x1, x2;
          split3(S[h][s][e], x0, x1, x2);
          bh[h][e] = x0;
          bm[h][e] = x1;
          bl[h][e] = x2;
        }
      // the six part products, smallest first, over four independent accumulators
#define QDR_P4(AP, BP)                                                   \
  P[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k##AP, BP[0], P[0], 0, 0, 0); \
  P[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k##AP, BP[1], P[1], 0, 0, 0); \
  Q[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q##AP, BP[0], Q[0], 0, 0, 0); \
  Q[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q##AP, BP[1], Q[1], 0, 0, 0);
      QDR_P4(l, bh)
      QDR_P4(h, bl)
      QDR_P4(m, bm)
      QDR_P4(m, bh)
      QDR_P4(h, bm)
      QDR_P4(h, bh)
#undef QDR_P4
    }
    if (!safe) {
      // running products of the gates from memory over logical channels 32w..32w+31:
      // lane (i = rg, t = 4jg + r)
      const int i = rg, ti = t0 + i;
#pragma unroll 1
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * jg + r, tt = t0 + t;
        float sa = 0.0f, sb = 0.0f;
        if (t >= i && tt < T) {
          for (int j = 32 * w; j < 32 * w + 32; ++j) {
            float x = A.k[(size_t)ti * ts + uo + j];
            for (int q = i + 1; q <= t; ++q)
              x *= (GATE == KDA) ? A.a[(size_t)(t0 + q) * ts + uo + j]
                                 : A.a[(size_t)(t0 + q) * A.n_unit + u];
            sa = fmaf(x, A.k[(size_t)tt * ts + uo + j], sa);
            sb = fmaf(x, A.q[(size_t)tt * ts + uo + j], sb);
          }
        }
        DA[r] = sa;
        DB[r] = sb;
      }
    }
    if (t0 + kCB < T) issue(t0 + kCB, pf);
    // partials D[t = 4jg + r][i = rg]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      L.gp[w][0][4 * jg + r][rg] = DA[r];
      L.gp[w][1][4 * jg + r][rg] = DB[r];
    }
    block_sync();

    // B2. the wave's Grams (-b_t A_ti for i < t, B_ti for i <= t; partials summed in a
    //     fixed order) and x_t = b_t (v_t - S_r (gam_t k_t)) for the lane's tokens
    float(*nL)[kCB] = reinterpret_cast<ChunkPriv*>(&L.kpl[0][0][0])[w].g[0];
    float(*gB)[kCB] = reinterpret_cast<ChunkPriv*>(&L.kpl[0][0][0])[w].g[1];
    float(*xw)[32] = reinterpret_cast<ChunkX*>(&L.kmi[0][0][0])[w].x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane + 64 * k, t = e >> 4, i = e & 15;
      const float sa = ((L.gp[0][0][t][i] + L.gp[1][0][t][i]) + L.gp[2][0][t][i]) + L.gp[3][0][t][i];
      const float sb = ((L.gp[0][1][t][i] + L.gp[1][1][t][i]) + L.gp[2][1][t][i]) + L.gp[3][1][t][i];
      nL[t][i] = (i < t) ? -L.bb[t] * sa : 0.0f;
      gB[t][i] = (i <= t) ? sb : 0.0f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * jg + r;
        xw[t][16 * h + rg] = L.bb[t] * (vcur[4 * h + r] - P[h][r]);
      }
    wave_sync_lds();

    // B3. deltas: (I + L) delta = x by forward substitution, one lane per row of the
    //     wave (column-oriented: the updates of one step are independent)
    if (lane < 32) {
      float d[kCB];
#pragma unroll
      for (int t = 0; t < kCB; ++t) d[t] = xw[t][lane];
#pragma unroll
      for (int i = 0; i < kCB - 1; ++i)
#pragma unroll
        for (int t = i + 1; t < kCB; ++t) d[t] = fmaf(nL[t][i], d[i], d[t]);
#pragma unroll
      for (int t = 0; t < kCB; ++t) xw[t][lane] = d[t];
    }
    wave_sync_lds();

    // B4. readouts o = S_r (gam q) + B delta on the matrix cores (A = B, B = deltas,
    //     C = S_r (gam q) in the output layout)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * w + 16 * h + rg;
      f32x4 acc = Q[h];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(gB[m][4 * ks + jg], xw[4 * ks + jg][16 * h + rg],
                                                   acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * jg + r;
        if (t0 + t < T) A.o[(size_t)(t0 + t) * ts + uo + row] = acc[r];
      }
    }

    // B5. S <- S diag(gam_end) + sum_t delta_t kt_t^T on the matrix cores. The k index
    //     runs over two copies of the 16 tokens so that one 16x16x32 step adds two of
    //     the six part products: A = positions x [part X | part Y] (LDS), B = the
    //     lane's deltas of tokens 8 (jg & 1) + e, C = state.
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ge = L.gend[32 * s + 8 * jg + e];
        S[0][s][e] *= ge;
        S[1][s][e] *= ge;
      }
    const bool lo_k = jg < 2;
    const int tk = 8 * (jg & 1);
    bf16x8 d1[2], d2[2], d3[2];  // B operands of the three steps
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 dh, dm, dl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 x0, x1, x2;
        split3(xw[tk + e][16 * h + rg], x0, x1, x2);
        dh[e] = x0;
        dm[e] = x1;
        dl[e] = x2;
      }
      d1[h] = dh;                // [dh ; dh]
      d2[h] = dm;                // [dm ; dm]
      d3[h] = lo_k ? dh : dl;    // [dh ; dl]
    }
    const int p12 = lo_k ? 0 : 1, p3 = lo_k ? 2 : 0;  // A parts: [h | m], [l | h]
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a12[2], a3[2];
#pragma unroll
      for (int bq = 0; bq < 2; ++bq) {
        const int pos = 32 * s + 8 * (m >> 2) + 4 * bq + (m & 3);
        a12[bq] = *reinterpret_cast<const bf16x8*>(&L.ktl[p12][pos][tk]);
        a3[bq] = *reinterpret_cast<const bf16x8*>(&L.ktl[p3][pos][tk]);
      }
      f32x4 c[2][2];
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c[bq][h] = (f32x4){S[h][s][4 * bq], S[h][s][4 * bq + 1], S[h][s][4 * bq + 2],
                             S[h][s][4 * bq + 3]};
      // three steps over four independent accumulators
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c[bq][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3[bq], d3[h], c[bq][h], 0, 0, 0);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c[bq][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a12[bq], d2[h], c[bq][h], 0, 0, 0);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c[bq][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a12[bq], d1[h], c[bq][h], 0, 0, 0);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[h][s][4 * bq + e] = c[bq][h][e];
    }
  }
  block_sync();

  if (A.m > 0)
    comp_select<ChunkLayout>(*reinterpret_cast<float(*)[64]>(&S[0][0][0]), A.m,
                             A.tok_idx + (size_t)u * A.m, A.tok_val + (size_t)u * A.m,
                             *reinterpret_cast<CompLds*>(&L.qpl[0][0][0]), L.jperm);

  // refit + requantize (the decode step's rule). Key-row absmax: the lane's two rows, the
  // 16 lanes of its DPP row (same positions), then the four waves.
  float* scr = reinterpret_cast<float*>(&L.kpl[0][0][0]);
  float* kmax = scr;             // [4][128]
  float* invA = scr + 4 * kD;    // [128]
  float* invc = scr + 5 * kD;    // [128]
  float* cpart = scr + 6 * kD;   // [4][128]
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t mx = row16_max_u32(__float_as_uint(fmaxf(fabsf(S[0][s][e]), fabsf(S[1][s][e]))));
      if (rg == 0) kmax[w * kD + 32 * s + 8 * jg + e] = __uint_as_float(mx);
    }
  block_sync();
  if (tid < kD) {
    const int p = tid;
    const float Am = fmaxf(fmaxf(kmax[p], kmax[kD + p]), fmaxf(kmax[2 * kD + p], kmax[3 * kD + p]));
    const float Aa = (Am == 0.0f) ? 1.0f : Am;
    const int bits = (int)((cur.sb >> (8 * (p >> 5))) & 0xFFu);
    A.Rs[uo + p] = div_qmax(Aa, bits);
    invA[p] = recip_rn(Aa);
  }
  block_sync();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float cm = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = S[h][s][e] * invA[32 * s + 8 * jg + e];
        S[h][s][e] = y;
        cm = fmaxf(cm, fabsf(y));
      }
    cpart[jg * kD + 32 * w + 16 * h + rg] = cm;
  }
  block_sync();
  if (tid < kD) {
    const int i = tid;
    float cm = fmaxf(fmaxf(cpart[i], cpart[kD + i]), fmaxf(cpart[2 * kD + i], cpart[3 * kD + i]));
    if (cm == 0.0f) cm = 1.0f;
    A.Cs[uo + i] = cm;
    invc[i] = recip_rn(cm);
  }
  block_sync();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const Seg sg = seg_from(cur.sb, s);
    uint8_t* seg = A.packed + cur.toff + sg.off;
    const float qmax = (float)((1 << (sg.bits - 1)) - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * w + 16 * h + rg;
      const float M = qmax * invc[row];
      QDR_WIDTH_DISPATCH(0, sg.bits, (requant_row<BB>(seg, row, jg, S[h][s], M)));
    }
  }
}

// S += tokens (one thread per token slot)
__global__ void __launch_bounds__(64) k_comp_add(int m, const uint16_t* tok_idx,
                                                 const float* tok_val, float* S) {
  const int t = threadIdx.x;
  const size_t u = blockIdx.x;
  if (t >= m) return;
  const uint32_t ix = tok_idx[u * m + t];
  if (ix >= (uint32_t)(kD * kD)) return;  // empty slot
  S[u * kD * kD + ix] += tok_val[u * m + t];
}

// persistent grid of each decode-step variant, per device (occupancy x CU count)
constexpr int kMaxDevices = 64;
int g_step_grid[kMaxDevices][2][2][3] = {};

}  // namespace

hipError_t launch_init(const Pool& p, uint8_t* packed, float* rs, float* cs, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  hipLaunchKernelGGL(k_init, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                     p.req_bytes, packed, rs, cs);
  return hipGetLastError();
}

hipError_t launch_quantize(const Pool& p, const float* S, uint8_t* packed, float* rs, float* cs,
                           hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                     p.req_bytes, S, packed, rs, cs, p.rule);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Pool& p, const uint8_t* packed, const float* rs,
                             const float* cs, float* S, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequantize, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                     p.req_bytes, packed, rs, cs, S);
  return hipGetLastError();
}

// Persistent grid size: resident groups per CU (occupancy query) x CUs, capped by the
// number of units. Queried once per process and kernel variant (one device per
// process assumed for the cache; the value only sizes the grid, correctness does not
// depend on it).
template <int GATE, bool UNIFORM, int RULE>
static int step_grid(int n_unit) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int& g = g_step_grid[dev >= 0 && dev < kMaxDevices ? dev : 0][GATE][UNIFORM ? 1 : 0][RULE];
  if (g == 0) {
    int cus = 0, per_cu = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<GATE, UNIFORM, RULE>,
                                                       kThreads, 0);
    g = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
  }
  return n_unit < g ? n_unit : g;
}

template <int GATE, bool UNIFORM, int RULE>
static void launch_step_rule(const StepArgs& A, hipStream_t s) {
  hipLaunchKernelGGL((k_step<GATE, UNIFORM, RULE>), dim3(step_grid<GATE, UNIFORM, RULE>(A.n_unit)),
                     dim3(kThreads), 0, s, A);
}

template <int GATE, bool UNIFORM>
static void launch_step_variant(const StepArgs& A, int rule, hipStream_t s) {
  if (rule == RULE_KEYROW) launch_step_rule<GATE, UNIFORM, RULE_KEYROW>(A, s);
  else if (rule == RULE_TENSOR) launch_step_rule<GATE, UNIFORM, RULE_TENSOR>(A, s);
  else launch_step_rule<GATE, UNIFORM, RULE_STEP>(A, s);
}

hipError_t launch_step(const Pool& p, int gate, uint8_t* packed, float* rs, float* cs,
                       const float* q, const float* k, const float* v, const float* a,
                       const float* b, float* o, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  StepArgs A{p.meta, p.n_head, p.n_unit / p.n_head, p.n_unit, p.req_bytes, p.uniform,
             {p.n_class[0], p.n_class[1], p.n_class[2]}, packed, rs, cs, q, k, v, a, b, o};
  if (gate == GDN) {
    if (p.uniform) launch_step_variant<GDN, true>(A, p.rule, s);
    else launch_step_variant<GDN, false>(A, p.rule, s);
  } else {
    if (p.uniform) launch_step_variant<KDA, true>(A, p.rule, s);
    else launch_step_variant<KDA, false>(A, p.rule, s);
  }
  return hipGetLastError();
}

// the width of a pool whose heads all have one width, else 0: such a pool's tiles sit at
// h * req_bytes / n_head, in key order (a single-width head keeps the logical order)
static int uniform_width(const Pool& p) {
  static const int widths[3] = {8, 6, 4};
  if (p.uniform)
    for (int c = 0; c < 3; ++c)
      if (p.n_class[c] == p.n_head) return widths[c];
  return 0;
}

hipError_t launch_window(const Pool& p, int gate, int W, int t, uint8_t* packed, float* rs,
                         float* cs, uint8_t* buf, const float* q, const float* k, const float* v,
                         const float* a, const float* b, float* o, int m, uint16_t* tok_idx,
                         float* tok_val, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  WinArgs A{p.meta, p.n_head, W, t, p.req_bytes, packed, rs, cs, buf, q, k, v, a, b, o,
            m, tok_idx, tok_val, uniform_width(p)};
  const bool small = W <= 64;
  if (gate == GDN) {
    if (small) hipLaunchKernelGGL((k_window_token<GDN, 64>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    else hipLaunchKernelGGL((k_window_token<GDN, kWinMax>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    if (t == W - 1) {
      if (m > 0) hipLaunchKernelGGL((k_window_fold<GDN, true>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
      else hipLaunchKernelGGL((k_window_fold<GDN, false>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    }
  } else {
    if (small) hipLaunchKernelGGL((k_window_token<KDA, 64>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    else hipLaunchKernelGGL((k_window_token<KDA, kWinMax>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    if (t == W - 1) {
      if (m > 0) hipLaunchKernelGGL((k_window_fold<KDA, true>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
      else hipLaunchKernelGGL((k_window_fold<KDA, false>), dim3(p.n_unit), dim3(kThreads), 0, s, A);
    }
  }
  return hipGetLastError();
}

hipError_t launch_chunk(const Pool& p, int gate, int T, uint8_t* packed, float* rs, float* cs,
                        const float* q, const float* k, const float* v, const float* a,
                        const float* b, float* o, int m, uint16_t* tok_idx, float* tok_val,
                        const float* S_in, hipStream_t s) {
  if (p.n_unit == 0 || (T == 0 && !S_in)) return hipSuccess;
  const int ubits = uniform_width(p);
  ChunkArgs A{p.meta, p.n_head, p.n_unit, T, p.req_bytes, packed, rs, cs, q, k, v, a, b, o,
              m, tok_idx, tok_val, S_in, ubits};
  if (gate == GDN) hipLaunchKernelGGL(k_chunk<GDN>, dim3(p.n_unit), dim3(kThreads), 0, s, A);
  else hipLaunchKernelGGL(k_chunk<KDA>, dim3(p.n_unit), dim3(kThreads), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_comp_add(int n_unit, int m, const uint16_t* tok_idx, const float* tok_val,
                           float* S, hipStream_t s) {
  if (n_unit == 0 || m == 0) return hipSuccess;
  hipLaunchKernelGGL(k_comp_add, dim3(n_unit), dim3(64), 0, s, m, tok_idx, tok_val, S);
  return hipGetLastError();
}

}  // namespace qdr
