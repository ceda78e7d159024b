// qdr_damp.hip -- gfx950 kernels of the DAMP-style storage variant (freedom251 page,
// section "DAMP: accuracy depends on the task": selected key channels kept in FP16, the
// others in INT8 with stochastic rounding).
//
// Per unit: half[128 rows][16] binary16 (the selected key channels, physical positions
// 0..15), codes[128 rows][112] int8 (the other channels, positions 16..127), R[112] fp32
// (one range per key row). perm[h][p] is the logical key channel at physical position p.
//
// Arithmetic contract (shared with the scalar reference, bit for bit):
//   gate + dequantize  S'_ip = fl(f32(h_ip) * g_p) (p < 16), fl(code_ip * fl(g_p * R_p))
//   u_i                fl32(s0 + s1), s0 and s1 the fp64 sums of S'_ip k_p over positions
//                      0..63 and 64..127, each in position order
//   delta / update     w_i = fl(b fl(v_i - u_i)), S_new = fma(w_i, k_p, S'_ip)
//   readout            o_i from S_new and q as u_i from S' and k
//   requantize         p < 16: binary16, round to nearest even; p >= 16: A_p = max_i
//                      |S_ip| (1 if 0), R_p = fl(A_p/127), y = fl(S * fl(1/A_p)),
//                      code = clamp(floor(y*127 + u), +-127) in fp64, u in [0, 1) = top 24
//                      bits of word p%4 of the Philox4x32-10 block for the counter
//                      (i*32 + p/4, unit, step lo, step hi) and key (seed lo, seed hi).
//
// Work decomposition: one work-group of 256 threads per unit. Thread t holds value row
// t >> 1 at the 64 positions of half t & 1 in registers (the fp64 half sums of the
// prediction and the readout are then in-thread and in position order); the key-row
// absmax is a shuffle reduce-scatter over the wave's 32 rows, then a max over the four
// waves through LDS. LDS holds only the input vectors and the ranges (3.5 KB).
#include "qdr_internal.h"

namespace qdr {
namespace {

constexpr int GDN = 0;
constexpr int KDA = 1;
constexpr int kH = kDampHalf;     // binary16 channels
constexpr int kI = kD - kDampHalf;  // INT8 channels

struct DampLds {
  double kd[kD], qd[kD];  // k, q in fp64 for the dot products
  float kp[kD], cf[kD];
  float invA[kD];
  float part[4][kD];  // per-wave key-row absmax
};

// a ^ b ^ k in one gfx950 three-input bit operation (truth table 0x96), k uniform
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC11): ten rounds of two 32x32 -> 64-bit
// products on the counter, the key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
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

// Max over the 32 rows of the wave that share this lane's half, for each of the lane's 64
// positions, as a reduce-scatter over lane bits 5..1: lane l ends with the positions
// off + 0 and off + 1 of its half, off = 32 b5 + 16 b4 + 8 b3 + 4 b2 + 2 b1.
__device__ __forceinline__ void half_colmax(const float (&a)[64], int lane, float& m0, float& m1,
                                            int& off) {
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j)
    x[j] = fmaxf(b5 ? a[j + 32] : a[j], __shfl_xor(b5 ? a[j] : a[j + 32], 32));
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    y[j] = fmaxf(b4 ? x[j + 16] : x[j], __shfl_xor(b4 ? x[j] : x[j + 16], 16));
  float z[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = fmaxf(b3 ? y[j + 8] : y[j], __shfl_xor(b3 ? y[j] : y[j + 8], 8));
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = fmaxf(b2 ? z[j + 4] : z[j], __shfl_xor(b2 ? z[j] : z[j + 4], 4));
  m0 = fmaxf(b1 ? v[2] : v[0], __shfl_xor(b1 ? v[0] : v[2], 2));
  m1 = fmaxf(b1 ? v[3] : v[1], __shfl_xor(b1 ? v[1] : v[3], 2));
  off = 32 * (int)b5 + 16 * (int)b4 + 8 * (int)b3 + 4 * (int)b2 + 2 * (int)b1;
}

// Row i's half-row pointers: raw code words q = 0..3 hold the codes of positions
// p0 + 16q .. p0 + 16q + 15 (for half 0, word 0 would be the binary16 positions: unused).
__device__ __forceinline__ int8_t* code_word(int8_t* crow, int seg, int q) {
  return crow + (seg ? 48 + 16 * q : 16 * (q - 1));
}

// floor(127 y + r 2^-24) clamped to [-127, 127]. Scaled by 2^24 it is
// floor(127 2^24 y + r) >> 24 (floor of a floor quotient), and 127 2^24 y + r is one fp64
// fma with the same single rounding as the unscaled fp64 sum (exact for |y| >= 2^-23; no
// integer is crossed below that); y is clamped to [-1, 1] first, which leaves the clamped
// result unchanged and keeps the floor inside int32. sr_scaled returns the scaled floor;
// the code is its top byte (>> 24).
__device__ __forceinline__ int sr_scaled(float y, uint32_t r24) {
  const float yc = fminf(fmaxf(y, -1.0f), 1.0f);
  return (int)floor(fma((double)yc, 2130706432.0, (double)r24));  // 127 * 2^24
}

// ranges and requantization of the register-held half rows, stored in place
__device__ __forceinline__ void damp_requant(DampLds& L, const DampArgs& A, int u,
                                             float (&Sr)[64]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = tid >> 1, seg = tid & 1, p0 = 64 * seg;
  {
    float ab[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) ab[e] = fabsf(Sr[e]);
    float m0, m1;
    int off;
    half_colmax(ab, lane, m0, m1, off);
    L.part[w][p0 + off] = m0;
    L.part[w][p0 + off + 1] = m1;
  }
  __syncthreads();
  if (tid < kD && tid >= kH) {
    const int p = tid;
    const float m = fmaxf(fmaxf(L.part[0][p], L.part[1][p]), fmaxf(L.part[2][p], L.part[3][p]));
    const float Aa = (m == 0.0f) ? 1.0f : m;
    A.R[(size_t)u * kI + (p - kH)] = Aa / 127.0f;
    L.invA[p] = 1.0f / Aa;
  }
  __syncthreads();
  const uint32_t k0 = (uint32_t)A.seed, k1 = (uint32_t)(A.seed >> 32);
  const uint32_t s0 = (uint32_t)A.step, s1 = (uint32_t)(A.step >> 32);
  if (seg == 0) {
    uint32_t hw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      hw[e] = (uint32_t)f16_bits(Sr[2 * e]) | ((uint32_t)f16_bits(Sr[2 * e + 1]) << 16);
    uint4* dst = reinterpret_cast<uint4*>(A.half + ((size_t)u * kD + i) * kH);
    dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dst[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
  }
  // the row's 112 INT8 positions split 56/56 over the pair: half 0 takes 16..71 (64..71
  // from its partner's registers), half 1 takes 72..127; 14 Philox blocks each
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __shfl_xor(Sr[e], 1);
  const int base = seg ? 72 : kH;
  uint32_t wd[14];
#pragma unroll
  for (int b = 0; b < 14; ++b) {
    const uint4 r = philox4x32_10((uint32_t)(i * 32 + base / 4 + b), (uint32_t)u, s0, s1, k0, k1);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
    // the codes are the top bytes of the scaled floors: byte selects pack four
    uint32_t t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * b + e;  // position base + j
      const float sv = seg ? Sr[8 + j] : (j < 48 ? Sr[16 + j] : x[j - 48]);
      const float y = sv * L.invA[base + j];
      t[e] = (uint32_t)sr_scaled(y, rw[e] >> 8);
    }
    wd[b] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(t[3], t[2], 0x0C0C0703u),
                                  __builtin_amdgcn_perm(t[1], t[0], 0x0C0C0703u), 0x05040100u);
  }
  int8_t* crow = A.codes + ((size_t)u * kD + i) * kI;
  if (seg == 0) {
    uint4* d = reinterpret_cast<uint4*>(crow);
    d[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    d[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    d[2] = make_uint4(wd[8], wd[9], wd[10], wd[11]);
    *reinterpret_cast<uint2*>(crow + 48) = make_uint2(wd[12], wd[13]);
  } else {
    *reinterpret_cast<uint2*>(crow + 56) = make_uint2(wd[0], wd[1]);
    uint4* d = reinterpret_cast<uint4*>(crow + 64);
    d[0] = make_uint4(wd[2], wd[3], wd[4], wd[5]);
    d[1] = make_uint4(wd[6], wd[7], wd[8], wd[9]);
    d[2] = make_uint4(wd[10], wd[11], wd[12], wd[13]);
  }
}

template <int GATE>
__global__ void __launch_bounds__(kThreads) k_damp_step(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const size_t uo = (size_t)u * kD;
  if (tid < kD) {
    const int p = tid, j = A.perm[(size_t)h * kD + p];
    const float kv = A.k[uo + j];
    L.kp[p] = kv;
    L.kd[p] = kv;
    L.qd[p] = A.q[uo + j];
    const float g = (GATE == KDA) ? A.a[uo + j] : A.a[u];
    L.cf[p] = p < kH ? g : g * A.R[(size_t)u * kI + (p - kH)];
  }
  const int i = tid >> 1, seg = tid & 1, p0 = 64 * seg;
  // this thread's half row: binary16 words (half 0) and code words
  uint4 raw[4], hraw[2];
  const int8_t* crow = A.codes + (uo + i) * kI;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    raw[q] = (q == 0 && seg == 0) ? make_uint4(0, 0, 0, 0)
                                  : *reinterpret_cast<const uint4*>(code_word(const_cast<int8_t*>(crow), seg, q));
  if (seg == 0) {
    const uint4* hr = reinterpret_cast<const uint4*>(A.half + (uo + i) * kH);
    hraw[0] = hr[0];
    hraw[1] = hr[1];
  } else {
    hraw[0] = hraw[1] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  // gated dequantization into registers
  float Sr[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    const uint4 x = raw[e >> 4];
    const uint32_t word = ((e >> 2) & 3) == 0 ? x.x : (((e >> 2) & 3) == 1 ? x.y : (((e >> 2) & 3) == 2 ? x.z : x.w));
    const float c = (float)(int8_t)(word >> (8 * (e & 3)));
    if (e < kH) {
      const uint4 hx = hraw[e >> 3];
      const int hq = (e >> 1) & 3;
      const uint32_t hw = hq == 0 ? hx.x : (hq == 1 ? hx.y : (hq == 2 ? hx.z : hx.w));
      const float hv = f16_value((uint16_t)(hw >> (16 * (e & 1))));
      Sr[e] = (seg == 0 ? hv : c) * L.cf[p0 + e];
    } else {
      Sr[e] = c * L.cf[p0 + e];
    }
  }
  // u_i: this thread's fp64 half sum in position order (a product of two fp32 values is exact
  // in fp64, so each fma adds exactly the product), the pair combined as s0 + s1
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 64; ++e) s = fma((double)Sr[e], L.kd[p0 + e], s);
  const double so = __shfl_xor(s, 1);
  const float uu = (float)(seg ? so + s : s + so);
  const float w = A.b[u] * (A.v[uo + i] - uu);
  double t = 0.0;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    Sr[e] = fmaf(w, L.kp[p0 + e], Sr[e]);
    t = fma((double)Sr[e], L.qd[p0 + e], t);
  }
  const double to = __shfl_xor(t, 1);
  if (seg == 0) A.o[uo + i] = (float)(t + to);
  damp_requant(L, A, u, Sr);
}

__global__ void __launch_bounds__(kThreads) k_damp_quantize(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const int i = tid >> 1, seg = tid & 1, p0 = 64 * seg;
  const float* Si = A.S + ((size_t)u * kD + i) * kD;
  const uint8_t* perm = A.perm + (size_t)h * kD;
  float Sr[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) Sr[e] = Si[perm[p0 + e]];
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
  DampArgs A{p.perm, p.n_head, p.gate, half, codes, R, q, k, v, a, b, o, S, Sout, seed, step};
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
