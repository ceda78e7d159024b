// qdr_damp.hip -- gfx950 kernels of the DAMP-style storage variant (freedom251 page,
// section "DAMP: accuracy depends on the task": selected key channels kept in FP16, the
// others in INT8 with stochastic rounding).
//
// Per unit: half[128 rows][16] binary16 (the selected key channels, physical positions
// 0..15), codes[128 rows][112] int8 (the other channels, positions 16..127), R[112] fp32
// (one range per key row). perm[h][p] is the logical key channel at physical position p.
//
// Arithmetic (the scalar reference's, except for the order of the fp64 dot products):
//   gate + dequantize  S'_ip = fl(f32(h_ip) * g_p) (p < 16), fl(code_ip * fl(g_p * R_p))
//   u_i                fl32 of the fp64 sum of S'_ip k_p; each product is exact in fp64,
//                      summed here as two half sums (each thread's 64 positions in register
//                      order, see dpos) added, where the reference takes one sum in key
//                      channel order: the fp32 results can differ on rare rounding ties
//   delta / update     w_i = fl(b fl(v_i - u_i)), S_new = fma(w_i, k_p, S'_ip)
//   readout            o_i = S_new q summed in fp32 (it feeds nothing back into the state;
//                      within the readout tolerance of the reference's fp64 sum)
//   requantize         p < 16: binary16, round to nearest even; p >= 16: A_p = max_i
//                      |S_ip| (1 if 0), R_p = fl(A_p/127), y = fl(S * fl(1/A_p)),
//                      code = clamp(floor(y*127 + u), +-127) exactly, u in [0, 1) = byte
//                      p%16 (little-endian over the words) of the Philox4x32-7 block for
//                      the counter (i*8 + p/16, unit, step lo, step hi) and key (seed lo,
//                      seed hi), times 2^-8.
//
// Work decomposition: one work-group of 256 threads per unit. Thread t holds 64 positions
// of value row t >> 1 in registers, half s = t & 1 of the row's positions (dpos): 8
// binary16 positions, 48 INT8 positions that make three whole Philox blocks and the half
// of block 4 that the thread codes, so that both threads of a row do the same work (the
// fp64 half sums of the prediction and the readout are in-thread); the key-row absmax is a
// shuffle reduce-scatter over the wave's 32 rows, then a max over the four waves through
// LDS. LDS holds only the input vectors, those maxima and the ranges (5.6 KB).
#include "qdr_internal.h"

namespace qdr {
namespace {

constexpr int GDN = 0;
constexpr int KDA = 1;
constexpr int kH = kDampHalf;     // binary16 channels
constexpr int kI = kD - kDampHalf;  // INT8 channels

// Per-position vectors in LDS. The two threads of a row read the positions of one register
// at once, 8 or 64 apart (dpos); 16 bytes of padding after position 63 put positions 64
// apart on different banks (without it, 512 bytes apart, every such read is a bank
// conflict).
constexpr int kPadF = 4;  // floats
constexpr int kPadD = 2;  // doubles
__device__ __forceinline__ int fidx(int p) { return p + (p >> 6) * kPadF; }
__device__ __forceinline__ int didx(int p) { return p + (p >> 6) * kPadD; }

// Physical position of register e of a thread of half s: registers 0..7 hold the binary16
// positions 8 s + e; 8..55 the INT8 positions 16..63 (s = 0) or 80..127 (s = 1), Philox
// blocks 1-3 or 5-7; 56..63 the positions 64..71 or 72..79, its half of block 4. Codes
// [0, 48) of the thread lie at byte 64 s of the row's 112, codes [48, 56) at byte 48 + 8 s.
__device__ __forceinline__ int dpos(int s, int e) {
  return e < 8 ? 8 * s + e : (e < 56 ? 8 + 64 * s + e : 8 + 8 * s + e);
}

struct DampLds {
  double kd[kD + kPadD];  // k in fp64 for the prediction
  float kp[kD + kPadF], qf[kD + kPadF], cf[kD + kPadF];
  float invA[kD + kPadF];
  float part[4][kD];  // per-wave key-row absmax
  int wide;           // some range of the unit outside [2^-126, 2^126]
};

// a ^ b ^ k in one gfx950 three-input bit operation (truth table 0x96), k uniform
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// Philox4x32-7 (Salmon, Moraes, Dror, Shaw, SC11): the published round function -- two
// 32x32 -> 64-bit products on the counter, the key advanced by the Weyl constants between
// rounds -- taken for seven rounds, the fewest with which the paper reports it passing its
// statistical batteries (its default of ten adds a safety margin).
__device__ __forceinline__ uint4 philox4x32_7(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 7; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = xor3(hi1, c1, k0);
    const uint32_t n2 = xor3(hi0, c3, k1);
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return make_uint4(c0, c1, c2, c3);
}

struct DampArgs {
  const uint8_t* perm;  // [n_head][128]
  int n_head, gate;
  int ident;  // perm is the identity for every head (no position-map load)
  uint16_t* half;
  int8_t* codes;
  float* R;
  const float* q;
  const float* k;
  const float* v;
  const float* a;
  const float* b;
  float* o;
  const float* S;  // quantize input [unit][128][128], logical order
  float* Sout;     // dequantize output, same layout
  uint64_t seed, step;
};

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // v_cvt_f16_f32, round to nearest even
}

__device__ __forceinline__ float f16_value(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Lane exchanges without LDS round trips: the value of lane ^ 1, ^ 2 (quad permutes) and
// ^ 8 (row rotation by 8 within each row of 16) by DPP moves; lane ^ 4 by a swizzle.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}
__device__ __forceinline__ double dpp_xor1(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), 0xB1, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// DPP forms on bit patterns (the float maxima below compare non-negative floats as
// unsigned integers: no NaN canonicalization, and the moves fuse into the max)
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_xor8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t swz_xor4(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x101F);
}

// max(|a|, |b|) in one instruction (source modifiers; no NaN canonicalization of the operands)
__device__ __forceinline__ uint32_t absmax2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_max_f32 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over the 32 rows of the wave that share this lane's half, for each of the lane's 64
// values in absolute value, as a reduce-scatter over lane bits 5..1: lane l ends with the
// positions off + 0 and off + 1 of its half, off = 32 b5 + 16 b4 + 8 b3 + 4 b2 + 2 b1.
// The values are exchanged in place and swapped back, so a is unchanged on return.
__device__ __forceinline__ void half_colmax(float (&a)[64], int lane, float& m0, float& m1,
                                            int& off) {
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  // Lane bits 5 and 4 by the gfx950 half-swaps: v_permlane32_swap exchanges the upper 32
  // lanes of its first operand with the lower 32 lanes of its second, so lanes 0-31 end
  // with both rows' values of position j and lanes 32-63 with those of j + 32, without
  // selects; v_permlane16_swap does the same within each half, for lane bit 4. From the
  // first level on the values are magnitudes, compared as bit patterns.
  uint32_t x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[j]), __float_as_uint(a[j + 32]),
                                                    false, false);
    x[j] = absmax2(r[0], r[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(r[0], r[1], false, false);
    a[j] = __uint_as_float(t[0]);
    a[j + 32] = __uint_as_float(t[1]);
  }
  uint32_t y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(x[j], x[j + 16], false, false);
    y[j] = max(r[0], r[1]);
  }
  uint32_t z[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = max(b3 ? y[j + 8] : y[j], dpp_xor8(b3 ? y[j] : y[j + 8]));
  uint32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = max(b2 ? z[j + 4] : z[j], swz_xor4(b2 ? z[j] : z[j + 4]));
  m0 = __uint_as_float(max(b1 ? v[2] : v[0], dpp_xor2(b1 ? v[0] : v[2])));
  m1 = __uint_as_float(max(b1 ? v[3] : v[1], dpp_xor2(b1 ? v[1] : v[3])));
  off = 32 * (int)((lane >> 5) & 1) + 16 * (int)((lane >> 4) & 1) + 8 * (int)b3 + 4 * (int)b2 +
        2 * (int)b1;
}

// Stochastic rounding: floor(127 y + r 2^-8) clamped to [-127, 127], r the row's random
// byte. Scaled by 2^8 it is floor((floor(127 2^8 y) + r) / 2^8): r is an integer, so it moves
// out of the inner floor, and the floor of a floor quotient is the floor of the quotient.
// y lies in [-1, 1] or is clamped to it (see damp_codes), which leaves the clamped result
// unchanged and keeps floor(127 2^8 y) + r inside [-32512, 32767]; the code is then its
// second byte (an arithmetic shift by 8).
__device__ __forceinline__ float sr_clamp(float y) { return fminf(fmaxf(y, -1.0f), 1.0f); }

// floor(32512 y) for four values y (32512 = 127 * 2^8), exactly: the products are rounded
// toward -inf (the MODE register's fp32 rounding field set to 2 around them, then back to
// nearest even), and the floor of the largest fp32 value <= x is floor(x), since every
// integer of this range is an fp32 value. Two wait states follow each mode write.
__device__ __forceinline__ void floor_scaled4(const float (&y)[4], int (&f)[4]) {
  asm("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 2\n\t"
      "s_nop 1\n\t"
      "v_mul_f32 %0, %8, %4\n\t"
      "v_mul_f32 %1, %8, %5\n\t"
      "v_mul_f32 %2, %8, %6\n\t"
      "v_mul_f32 %3, %8, %7\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1\n\t"
      "v_cvt_flr_i32_f32 %0, %0\n\t"
      "v_cvt_flr_i32_f32 %1, %1\n\t"
      "v_cvt_flr_i32_f32 %2, %2\n\t"
      "v_cvt_flr_i32_f32 %3, %3"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "s"(32512.0f));
}

// The INT8 codes of the thread's half row. With every range of the unit in [2^-126, 2^126],
// fl(1/A) is normal with relative error <= 2^-24, so |S fl(1/A)| <= 1 + 2^-24, which rounds
// to at most 1: y needs no clamp (CLAMP false). Otherwise y is clamped to [-1, 1].
template <bool CLAMP>
__device__ __forceinline__ void damp_codes(const DampLds& L, const DampArgs& A, int u,
                                           const float (&Sr)[64], uint32_t k0, uint32_t k1,
                                           uint32_t s0, uint32_t s1) {
  const int tid = threadIdx.x;
  const int i = tid >> 1, seg = tid & 1;
  auto clampy = [](float y) { return CLAMP ? sr_clamp(y) : y; };
  // The row's 112 INT8 positions in Philox blocks of 16 (one block per 16 positions), 56 per
  // thread: blocks 1-3 (half 0) or 5-7 (half 1) from registers 8..55, stored as 16 bytes per
  // block; block 4 (positions 64..79) is generated by both threads, each coding its 8
  // positions (registers 56..63), 8 bytes each.
  int8_t* crow = A.codes + ((size_t)u * kD + i) * kI;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int blk = seg ? 5 + b : 1 + b;  // positions 16 blk .. 16 blk + 15
    const uint4 r = philox4x32_7((uint32_t)(i * 8 + blk), (uint32_t)u, s0, s1, k0, k1);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
    uint32_t wd[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the codes are the second bytes of the scaled floors: byte selects pack four
      float yc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * q + e;  // position 16 blk + j, register 8 + 16 b + j
        yc[e] = clampy(Sr[8 + 16 * b + j] * L.invA[fidx(16 * blk + j)]);
      }
      int f[4];
      floor_scaled4(yc, f);
      uint32_t t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (uint32_t)(f[e] + (int)((rw[q] >> (8 * e)) & 0xFFu));
      wd[q] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(t[3], t[2], 0x0C0C0501u),
                                    __builtin_amdgcn_perm(t[1], t[0], 0x0C0C0501u), 0x05040100u);
    }
    *reinterpret_cast<uint4*>(crow + 16 * (blk - 1)) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  {
    const uint4 r = philox4x32_7((uint32_t)(i * 8 + 4), (uint32_t)u, s0, s1, k0, k1);
    const uint32_t rw[2] = {seg ? r.z : r.x, seg ? r.w : r.y};
    uint32_t wd[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float yc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * q + e;  // position 64 + 8 seg + j, register 56 + j
        yc[e] = clampy(Sr[56 + j] * L.invA[fidx(64 + 8 * seg + j)]);
      }
      int f[4];
      floor_scaled4(yc, f);
      uint32_t t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (uint32_t)(f[e] + (int)((rw[q] >> (8 * e)) & 0xFFu));
      wd[q] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(t[3], t[2], 0x0C0C0501u),
                                    __builtin_amdgcn_perm(t[1], t[0], 0x0C0C0501u), 0x05040100u);
    }
    *reinterpret_cast<uint2*>(crow + 48 + 8 * seg) = make_uint2(wd[0], wd[1]);
  }
}

// ranges and requantization of the register-held half rows, stored in place
__device__ __forceinline__ void damp_requant(DampLds& L, const DampArgs& A, int u,
                                             float (&Sr)[64]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = tid >> 1, seg = tid & 1;
  {
    float m0, m1;
    int off;
    half_colmax(Sr, lane, m0, m1, off);
    L.part[w][dpos(seg, off)] = m0;  // registers off, off + 1: adjacent positions
    L.part[w][dpos(seg, off) + 1] = m1;
  }
  if (tid == 0) L.wide = 0;
  __syncthreads();
  if (tid < kD && tid >= kH) {
    const int p = tid;
    const float m = fmaxf(fmaxf(L.part[0][p], L.part[1][p]), fmaxf(L.part[2][p], L.part[3][p]));
    const float Aa = (m == 0.0f) ? 1.0f : m;
    A.R[(size_t)u * kI + (p - kH)] = div_qmax(Aa, 8);  // Aa / 127
    L.invA[fidx(p)] = recip_rn(Aa);
    if (!(Aa >= 0x1p-126f && Aa <= 0x1p126f)) L.wide = 1;
  }
  __syncthreads();
  const uint32_t k0 = (uint32_t)A.seed, k1 = (uint32_t)(A.seed >> 32);
  const uint32_t s0 = (uint32_t)A.step, s1 = (uint32_t)(A.step >> 32);
  {
    uint32_t hw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      hw[e] = (uint32_t)f16_bits(Sr[2 * e]) | ((uint32_t)f16_bits(Sr[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(A.half + ((size_t)u * kD + i) * kH + 8 * seg) =
        make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
  const int wide = __builtin_amdgcn_readfirstlane(L.wide);
  if (wide) damp_codes<true>(L, A, u, Sr, k0, k1, s0, s1);
  else damp_codes<false>(L, A, u, Sr, k0, k1, s0, s1);
}

template <int GATE>
__global__ void __launch_bounds__(kThreads) k_damp_step(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const size_t uo = (size_t)u * kD;
  if (tid < kD) {
    const int p = tid;
    int j = p;
    if (!A.ident) j = A.perm[(size_t)h * kD + p];
    const float kv = A.k[uo + j];
    L.kp[fidx(p)] = kv;
    L.kd[didx(p)] = kv;
    L.qf[fidx(p)] = A.q[uo + j];
    const float g = (GATE == KDA) ? A.a[uo + j] : A.a[u];
    L.cf[fidx(p)] = p < kH ? g : g * A.R[(size_t)u * kI + (p - kH)];
  }
  const int i = tid >> 1, seg = tid & 1;
  // this thread's half row: 8 binary16 values and 56 codes (see dpos)
  const uint4 hraw = *reinterpret_cast<const uint4*>(A.half + (uo + i) * kH + 8 * seg);
  const int8_t* crow = A.codes + (uo + i) * kI;
  uint4 craw[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) craw[q] = *reinterpret_cast<const uint4*>(crow + 64 * seg + 16 * q);
  const uint2 caw = *reinterpret_cast<const uint2*>(crow + 48 + 8 * seg);
  __syncthreads();
  // gated dequantization into registers
  float Sr[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    float x;
    if (e < 8) {
      const int hq = e >> 1;
      const uint32_t hw = hq == 0 ? hraw.x : (hq == 1 ? hraw.y : (hq == 2 ? hraw.z : hraw.w));
      x = f16_value((uint16_t)(hw >> (16 * (e & 1))));
    } else if (e < 56) {
      const int c = e - 8, cq = (c >> 2) & 3;
      const uint4 cx = craw[c >> 4];
      const uint32_t word = cq == 0 ? cx.x : (cq == 1 ? cx.y : (cq == 2 ? cx.z : cx.w));
      x = (float)(int8_t)(word >> (8 * (c & 3)));
    } else {
      const int c = e - 56;
      x = (float)(int8_t)((c < 4 ? caw.x : caw.y) >> (8 * (c & 3)));
    }
    Sr[e] = x * L.cf[fidx(dpos(seg, e))];
  }
  // u_i: this thread's fp64 half sum in register order (a product of two fp32 values is
  // exact in fp64, so each fma adds exactly the product), the pair combined as s0 + s1
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 64; ++e) s = fma((double)Sr[e], L.kd[didx(dpos(seg, e))], s);
  const double so = dpp_xor1(s);
  const float uu = (float)(seg ? so + s : s + so);
  const float w = A.b[u] * (A.v[uo + i] - uu);
  // the readout feeds nothing back into the state, so it is summed in fp32 (two chains of
  // 32 fmas per thread; within the readout tolerance of the reference's fp64 sum)
  float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
  for (int e = 0; e < 64; e += 2) {
    Sr[e] = fmaf(w, L.kp[fidx(dpos(seg, e))], Sr[e]);
    Sr[e + 1] = fmaf(w, L.kp[fidx(dpos(seg, e + 1))], Sr[e + 1]);
    t0 = fmaf(Sr[e], L.qf[fidx(dpos(seg, e))], t0);
    t1 = fmaf(Sr[e + 1], L.qf[fidx(dpos(seg, e + 1))], t1);
  }
  const float t = t0 + t1;
  const float to = dpp_xor1(t);
  if (seg == 0) A.o[uo + i] = t + to;
  damp_requant(L, A, u, Sr);
}

__global__ void __launch_bounds__(kThreads) k_damp_quantize(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const int i = tid >> 1, seg = tid & 1;
  const float* Si = A.S + ((size_t)u * kD + i) * kD;
  const uint8_t* perm = A.perm + (size_t)h * kD;
  float Sr[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) Sr[e] = Si[perm[dpos(seg, e)]];
  damp_requant(L, A, u, Sr);
}

// readback S [unit][128][128] (logical order): f32(h) or fl(code * R)
__global__ void __launch_bounds__(kThreads) k_damp_dequantize(DampArgs A) {
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  float* Su = A.Sout + (size_t)u * kD * kD;
  const uint8_t* perm = A.perm + (size_t)h * kD;
  for (int e = tid; e < kD * kD; e += kThreads) {
    const int i = e >> 7, p = e & (kD - 1);
    const size_t r = (size_t)u * kD + i;
    Su[(size_t)i * kD + perm[p]] =
        p < kH ? f16_value(A.half[r * kH + p])
               : (float)A.codes[r * kI + (p - kH)] * A.R[(size_t)u * kI + (p - kH)];
  }
}

// zero state: codes 0, binary16 zeros, R = 1/127
__global__ void __launch_bounds__(kThreads) k_damp_init(DampArgs A) {
  const int tid = threadIdx.x, u = blockIdx.x;
  for (int e = tid; e < kD * kH; e += kThreads) A.half[(size_t)u * kD * kH + e] = 0;
  for (int e = tid; e < kD * kI; e += kThreads) A.codes[(size_t)u * kD * kI + e] = 0;
  if (tid < kI) A.R[(size_t)u * kI + tid] = 1.0f / 127.0f;
}

}  // namespace

hipError_t launch_damp(int op, const DampPool& p, uint16_t* half, int8_t* codes, float* R,
                       const float* q, const float* k, const float* v, const float* a,
                       const float* b, float* o, const float* S, float* Sout, uint64_t seed,
                       uint64_t step, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  DampArgs A{p.perm, p.n_head, p.gate, p.ident, half, codes, R, q, k, v, a, b, o, S, Sout, seed,
             step};
  const dim3 grid(p.n_unit), block(kThreads);
  switch (op) {
    case kDampInit: hipLaunchKernelGGL(k_damp_init, grid, block, 0, s, A); break;
    case kDampQuantize: hipLaunchKernelGGL(k_damp_quantize, grid, block, 0, s, A); break;
    case kDampDequantize: hipLaunchKernelGGL(k_damp_dequantize, grid, block, 0, s, A); break;
    default:
      if (p.gate == GDN) hipLaunchKernelGGL(k_damp_step<GDN>, grid, block, 0, s, A);
      else hipLaunchKernelGGL(k_damp_step<KDA>, grid, block, 0, s, A);
  }
  return hipGetLastError();
}

}  // namespace qdr
