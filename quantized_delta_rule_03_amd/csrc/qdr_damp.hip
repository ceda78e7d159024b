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
// Work decomposition: one work-group of 256 threads per unit; the fp32 state tile sits in
// LDS (rows padded against bank conflicts); thread t owns value row t >> 1 and the
// position half t & 1 for the dot products, the update and the requantization, and key
// row 16 + t (t < 112) for the range.
#include "qdr_internal.h"

namespace qdr {
namespace {

constexpr int GDN = 0;
constexpr int KDA = 1;
constexpr int kH = kDampHalf;     // binary16 channels
constexpr int kI = kD - kDampHalf;  // INT8 channels
constexpr int kP = kD + 4;        // LDS row pitch (floats)

struct DampLds {
  float S[kD][kP];
  float kp[kD], qp[kD], gp[kD], cf[kD];
  float invA[kD];
};

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
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
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

// key-row ranges over the tile and the requantized stores (the rows' owners)
__device__ void damp_requant(DampLds& L, const DampArgs& A, int u) {
  const int tid = threadIdx.x;
  {
    // column absmax: threads (position, row half), then the two halves
    const int p = tid & (kD - 1), r0 = (tid >> 7) * 64;
    float m = 0.0f;
    if (p >= kH)
      for (int i = r0; i < r0 + 64; ++i) m = fmaxf(m, fabsf(L.S[i][p]));
    if (tid >= kD) L.cf[p] = m;  // cf is dead by now: it holds the second halves
    __syncthreads();
    if (tid < kD && p >= kH) {
      m = fmaxf(m, L.cf[p]);
      const float Aa = (m == 0.0f) ? 1.0f : m;
      A.R[(size_t)u * kI + (p - kH)] = Aa / 127.0f;
      L.invA[p] = 1.0f / Aa;
    }
  }
  __syncthreads();
  const int i = tid >> 1, seg = tid & 1;
  const uint32_t k0 = (uint32_t)A.seed, k1 = (uint32_t)(A.seed >> 32);
  const uint32_t s0 = (uint32_t)A.step, s1 = (uint32_t)(A.step >> 32);
  if (seg == 0) {
    uint16_t hb[kH];
#pragma unroll
    for (int p = 0; p < kH; ++p) hb[p] = f16_bits(L.S[i][p]);
    uint4* dst = reinterpret_cast<uint4*>(A.half + ((size_t)u * kD + i) * kH);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(hb);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  // INT8 positions of this half: 16..63 (seg 0) or 64..127 (seg 1)
  const int p0 = seg ? 64 : kH, p1 = seg ? kD : 64;
  int8_t* crow = A.codes + ((size_t)u * kD + i) * kI;
  for (int pb = p0; pb < p1; pb += 16) {
    uint32_t pk[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int pq = pb + 4 * q4;
      const uint4 r = philox4x32_10((uint32_t)(i * 32 + pq / 4), (uint32_t)u, s0, s1, k0, k1);
      const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = pq + e;
        const float y = L.S[i][p] * L.invA[p];
        double t = floor((double)y * 127.0 + ldexp((double)(rw[e] >> 8), -24));
        t = fmin(fmax(t, -127.0), 127.0);
        word |= ((uint32_t)(uint8_t)(int8_t)(int)t) << (8 * e);
      }
      pk[q4] = word;
    }
    *reinterpret_cast<uint4*>(crow + (pb - kH)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

template <int GATE>
__global__ void __launch_bounds__(kThreads) k_damp_step(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const size_t uo = (size_t)u * kD;
  if (tid < kD) {
    const int p = tid, j = A.perm[(size_t)h * kD + p];
    L.kp[p] = A.k[uo + j];
    L.qp[p] = A.q[uo + j];
    const float g = (GATE == KDA) ? A.a[uo + j] : A.a[u];
    L.gp[p] = g;
    L.cf[p] = p < kH ? g : g * A.R[(size_t)u * kI + (p - kH)];
  }
  __syncthreads();
  const int i = tid >> 1, seg = tid & 1;
  const int p0 = seg * 64;
  // gated dequantization of this thread's 64 positions
  if (seg == 0) {
    const uint16_t* hr = A.half + (uo + i) * kH;
#pragma unroll
    for (int p = 0; p < kH; ++p) L.S[i][p] = f16_value(hr[p]) * L.cf[p];
  }
  {
    // this half's codes: 48 (seg 0) or 64 (seg 1) bytes, 16-byte aligned
    const uint4* cr = reinterpret_cast<const uint4*>(A.codes + (uo + i) * kI + (seg ? 64 - kH : 0));
    const int n16 = seg ? 4 : 3;
    const int pb = seg ? 64 : kH;
    for (int v16 = 0; v16 < n16; ++v16) {
      const uint4 x = cr[v16];
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int p = pb + 16 * v16 + e;
        const float c = (float)(int8_t)(xw[e >> 2] >> (8 * (e & 3)));
        L.S[i][p] = c * L.cf[p];
      }
    }
  }
  // u_i: this thread's fp64 half sum in position order, the pair combined as s0 + s1
  double s = 0.0;
  for (int p = p0; p < p0 + 64; ++p) s += (double)L.S[i][p] * (double)L.kp[p];
  const double so = __shfl_xor(s, 1);
  const float uu = (float)(seg ? so + s : s + so);
  const float w = A.b[u] * (A.v[uo + i] - uu);
  double t = 0.0;
  for (int p = p0; p < p0 + 64; ++p) {
    const float sn = fmaf(w, L.kp[p], L.S[i][p]);
    L.S[i][p] = sn;
    t += (double)sn * (double)L.qp[p];
  }
  const double to = __shfl_xor(t, 1);
  if (seg == 0) A.o[uo + i] = (float)(t + to);
  __syncthreads();
  damp_requant(L, A, u);
}

__global__ void __launch_bounds__(kThreads) k_damp_quantize(DampArgs A) {
  __shared__ __attribute__((aligned(16))) DampLds L;
  const int tid = threadIdx.x, u = blockIdx.x, h = u % A.n_head;
  const float* Su = A.S + (size_t)u * kD * kD;
  const uint8_t* perm = A.perm + (size_t)h * kD;
  for (int e = tid; e < kD * kD; e += kThreads) {
    const int i = e >> 7, p = e & (kD - 1);
    L.S[i][p] = Su[(size_t)i * kD + perm[p]];
  }
  __syncthreads();
  damp_requant(L, A, u);
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
