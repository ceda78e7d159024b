// qdr_kernels.hip -- gfx950 kernels of libqdr: init, quantize, dequantize, decode step.
//
// Work decomposition (all kernels): one work-group of 256 threads (4 wave64) per
// (request, head) unit. Wave w owns segment w of the tile, i.e. physical key positions
// 32w..32w+31, which all share one code width. Lane l of a wave owns value rows
// rg + 16 r (rg = l & 15, r = 0..7) at the 8 key positions 32w + 8 jg + m (jg = l >> 4,
// m = 0..7): 64 state entries per lane, held in VGPRs for the whole step.
//
// With that layout a wave-wide load of one row slot r reads 16 consecutive segment
// rows x 4 lanes, i.e. one contiguous 64*b-byte block (512 B at 8 bits); key-row
// (column) reductions stay inside a wave (16 lanes of one DPP row), value-row
// reductions go through LDS across the 16 (wave, jg) partials.
//
// Arithmetic contract (identical in every rounding to the scalar reference):
//   dequant + gate   P = fl(code * cf_j) as fma(field, cf_j, -bias*cf_j) (exact),
//                    S' = fl(P * rf_i)
//   prediction       u_i = fl32(rf_i * sum_j code_ij (cf_j k_j)) in fp64
//   delta            w_i = fl(b * fl(v_i - u_i)),  S_new = fma(w_i, k_j, S')
//   readout          o_i = sum_j S_new_ij q_j (fp32, fixed order)
//   refit            A_j = max_i |S_new_ij| (1 if 0), R_j = A_j / Qmax_j, invA = 1/A_j,
//                    y = fl(S_new * invA), c_i = max_j |y| (1 if 0), M = fl(Qmax * (1/c_i))
//   requant          field = RNE(y*M) + 2^(b-1), taken from fma(y, M, 2^23 + 2^(b-1))
//                    whose exact value lies in [2^23, 2^24) where the fp32 spacing is 1.
#include "qdr_internal.h"

namespace qdr {
namespace {

constexpr int GDN = 0;
constexpr int KDA = 1;

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

template <int B>
__device__ __forceinline__ Raw load_row(const uint8_t* seg, int row, int jg) {
  Raw r;
  if constexpr (B == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(seg + row * 32 + jg * 8);
    r.lo = x.x;
    r.hi = x.y;
  } else if constexpr (B == 4) {
    r.lo = *reinterpret_cast<const uint32_t*>(seg + row * 16 + jg * 4);
    r.hi = 0;
  } else {
    // 6 bytes at row*24 + 6*jg; read the two aligned dwords that contain them
    const int start = row * 24 + ((jg * 6) & ~3);
    const uint32_t* p = reinterpret_cast<const uint32_t*>(seg + start);
    uint32_t a0 = p[0], a1 = p[1];
    const int sh = ((jg * 6) & 3) * 8;  // 0 or 16
    const uint64_t x = ((uint64_t)a1 << 32 | a0) >> sh;
    r.lo = (uint32_t)x;
    r.hi = (uint32_t)(x >> 32);
  }
  return r;
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
#pragma unroll
    for (int m = 0; m < 8; ++m) f[m] = (float)((raw.lo >> (4 * m)) & 0xFu);
  } else {
    const uint64_t x = ((uint64_t)raw.hi << 32) | raw.lo;
#pragma unroll
    for (int m = 0; m < 8; ++m) f[m] = (float)((uint32_t)(x >> (6 * m)) & 0x3Fu);
  }
}

template <int B>
__device__ __forceinline__ void store_row(uint8_t* seg, int row, int jg, const uint32_t fld[8]) {
  if constexpr (B == 8) {
    uint2 x;
    x.x = fld[0] | (fld[1] << 8) | (fld[2] << 16) | (fld[3] << 24);
    x.y = fld[4] | (fld[5] << 8) | (fld[6] << 16) | (fld[7] << 24);
    *reinterpret_cast<uint2*>(seg + row * 32 + jg * 8) = x;
  } else if constexpr (B == 4) {
    uint32_t x = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) x |= fld[m] << (4 * m);
    *reinterpret_cast<uint32_t*>(seg + row * 16 + jg * 4) = x;
  } else {
    uint64_t x = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) x |= (uint64_t)fld[m] << (6 * m);
    uint8_t* dst = seg + row * 24 + jg * 6;
    if ((jg & 1) == 0) {  // 4-byte aligned start
      *reinterpret_cast<uint32_t*>(dst) = (uint32_t)x;
      *reinterpret_cast<uint16_t*>(dst + 4) = (uint16_t)(x >> 32);
    } else {              // 2-byte aligned start, dword at +2
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)x;
      *reinterpret_cast<uint32_t*>(dst + 2) = (uint32_t)(x >> 16);
    }
  }
}

template <int B>
__device__ __forceinline__ void load_tile_rows(const uint8_t* seg, int rg, int jg, Raw raw[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) raw[r] = load_row<B>(seg, rg + 16 * r, jg);
}

__device__ __forceinline__ void load_rows_dispatch(int B, const uint8_t* seg, int rg, int jg,
                                                   Raw raw[8]) {
  if (B == 8) load_tile_rows<8>(seg, rg, jg, raw);
  else if (B == 6) load_tile_rows<6>(seg, rg, jg, raw);
  else load_tile_rows<4>(seg, rg, jg, raw);
}

__device__ __forceinline__ void decode_dispatch(int B, Raw raw, float f[8]) {
  if (B == 8) decode_row<8>(raw, f);
  else if (B == 6) decode_row<6>(raw, f);
  else decode_row<4>(raw, f);
}

// requantize the lane's normalised entries y (8 rows x 8 positions) and store them
template <int B>
__device__ __forceinline__ void requant_store(uint8_t* seg, int rg, int jg, const float (&y)[8][8],
                                              const float (&M)[8]) {
  const float magic = 8388608.0f + (float)(1 << (B - 1));
  const uint32_t mask = (1u << B) - 1u;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t fld[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) fld[m] = __float_as_uint(fmaf(y[r][m], M[r], magic)) & mask;
    store_row<B>(seg, rg + 16 * r, jg, fld);
  }
}

__device__ __forceinline__ void requant_dispatch(int B, uint8_t* seg, int rg, int jg,
                                                 const float (&y)[8][8], const float (&M)[8]) {
  if (B == 8) requant_store<8>(seg, rg, jg, y, M);
  else if (B == 6) requant_store<6>(seg, rg, jg, y, M);
  else requant_store<4>(seg, rg, jg, y, M);
}

__device__ __forceinline__ float shfl_xor_f(float x, int d) { return __shfl_xor(x, d, 64); }

// Shared tail of quantize and decode step: refit both scale axes of the lane-held
// state s (overwritten by y) and write R (physical order) and c. Returns through
// LDS sinvc[] the reciprocal value-column scales. Contains block barriers: every
// thread of the block must call it.
struct TailLds {
  float invA[kD];
  float invc[kD];
  float cpart[16 * kD];
};

__device__ __forceinline__ void refit_tail(float (&s)[8][8], int w, int rg, int jg, int B,
                                           TailLds& L, float* __restrict__ Rs_u,
                                           float* __restrict__ Cs_u) {
  const int p0 = 32 * w + 8 * jg;
  // key-row absmax: in-lane over 8 rows, then across the 16 lanes rg of this jg
  float am[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    float x = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) x = fmaxf(x, fabsf(s[r][m]));
    am[m] = x;
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
    for (int m = 0; m < 8; ++m) am[m] = fmaxf(am[m], shfl_xor_f(am[m], d));
  }
  float Am = am[0];
#pragma unroll
  for (int m = 1; m < 8; ++m) Am = ((rg & 7) == m) ? am[m] : Am;
  if (rg < 8) {
    const float A = (Am == 0.0f) ? 1.0f : Am;
    const float qmax = (float)((1 << (B - 1)) - 1);
    Rs_u[p0 + rg] = A / qmax;
    L.invA[p0 + rg] = 1.0f / A;
  }
  __syncthreads();
  float ia[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) ia[m] = L.invA[p0 + m];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float cm = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float y = s[r][m] * ia[m];
      s[r][m] = y;
      cm = fmaxf(cm, fabsf(y));
    }
    L.cpart[(w * 4 + jg) * kD + rg + 16 * r] = cm;
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < kD) {
    float cm = 0.0f;
    for (int t = 0; t < 16; ++t) cm = fmaxf(cm, L.cpart[t * kD + tid]);
    if (cm == 0.0f) cm = 1.0f;
    Cs_u[tid] = cm;
    L.invc[tid] = 1.0f / cm;
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
  requant_dispatch(sg.bits, seg, rg, jg, y, M);
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
__global__ void __launch_bounds__(kThreads) k_quantize(const void* meta, int n_head,
                                                       uint32_t req_bytes, const float* S,
                                                       uint8_t* packed, float* Rs, float* Cs) {
  __shared__ TailLds L;
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
  refit_tail(s, w, rg, jg, sg.bits, L, Rs + uo, Cs + uo);
  __syncthreads();
  const float qmax = (float)((1 << (sg.bits - 1)) - 1);
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) M[rr] = qmax * L.invc[rg + 16 * rr];
  requant_dispatch(sg.bits, seg, rg, jg, s, M);
}

// ------------------------------------------------------------------------------
// dequantize: S_hat[i][j] = fl(fl(code * R_j) * c_i), logical order
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
  load_rows_dispatch(sg.bits, seg, rg, jg, raw);
  const size_t uo = (size_t)u * kD;
  const int p0 = 32 * w + 8 * jg;
  const float bias = (float)(1 << (sg.bits - 1));
  float R[8], nb[8];
  int col[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    R[m] = Rs[uo + p0 + m];
    nb[m] = -bias * R[m];
    col[m] = mh->identity ? p0 + m : (int)mh->perm[p0 + m];
  }
  float* Su = S + (size_t)u * kD * kD;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int i = rg + 16 * rr;
    const float c = Cs[uo + i];
    float f[8];
    decode_dispatch(sg.bits, raw[rr], f);
#pragma unroll
    for (int m = 0; m < 8; ++m) Su[(size_t)i * kD + col[m]] = fmaf(f[m], R[m], nb[m]) * c;
  }
}

// ------------------------------------------------------------------------------
// decode step
// ------------------------------------------------------------------------------
struct StepLds {
  double Kd[kD];       // cf_j * k_j in fp64, physical order
  float k[kD], q[kD], cf[kD];
  float rf[kD], v[kD], w[kD];
  union {
    double upart[16 * kD];  // per (wave, jg) partial of sum_j code_ij cf_j k_j
    struct {
      float opart[16 * kD];
      float spare[16 * kD];
    } f;
  } part;
  TailLds tail;
};

template <int GATE>
__global__ void __launch_bounds__(kThreads) k_step(const void* meta, int n_head,
                                                   uint32_t req_bytes, uint8_t* packed,
                                                   float* Rs, float* Cs, const float* q,
                                                   const float* k, const float* v,
                                                   const float* a, const float* b, float* o) {
  __shared__ StepLds L;
  const int u = blockIdx.x, r = u / n_head, h = u % n_head;
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = tid & 63, rg = lane & 15, jg = lane >> 4;
  const MetaHead* mh = meta_heads(meta) + h;
  const Seg sg = seg_of(mh, w);
  uint8_t* seg = packed + (size_t)r * req_bytes + mh->tile_off + sg.off;

  // 1. issue the code loads first so their latency overlaps the vector set-up
  Raw raw[8];
  load_rows_dispatch(sg.bits, seg, rg, jg, raw);

  const size_t uo = (size_t)u * kD;
  if (tid < kD) {
    const int p = tid;
    const int j = mh->identity ? p : (int)mh->perm[p];
    const float kk = k[uo + j], qq = q[uo + j], R = Rs[uo + p];
    const float cf = (GATE == KDA) ? a[uo + j] * R : R;
    L.k[p] = kk;
    L.q[p] = qq;
    L.cf[p] = cf;
    L.Kd[p] = (double)cf * (double)kk;
  } else {
    const int i = tid - kD;
    const float c = Cs[uo + i];
    L.rf[i] = (GATE == GDN) ? a[u] * c : c;
    L.v[i] = v[uo + i];
  }
  __syncthreads();

  // 2. dequantize + gate, partial prediction sums (fp64)
  const int p0 = 32 * w + 8 * jg;
  const float bias = (float)(1 << (sg.bits - 1));
  float cf[8], nb[8];
  double Kd[8];
  double kdsum = 0.0;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    cf[m] = L.cf[p0 + m];
    nb[m] = -bias * cf[m];
    Kd[m] = L.Kd[p0 + m];
    kdsum += Kd[m];
  }
  float s[8][8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int i = rg + 16 * rr;
    const float rf = L.rf[i];
    float f[8];
    decode_dispatch(sg.bits, raw[rr], f);
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float P = fmaf(f[m], cf[m], nb[m]);  // = fl((field - bias) * cf), exact rewrite
      s[rr][m] = P * rf;
      acc = fma((double)f[m], Kd[m], acc);
    }
    acc = fma(-(double)bias, kdsum, acc);
    L.part.upart[(w * 4 + jg) * kD + i] = acc;
  }
  __syncthreads();

  // 3. prediction u, delta w (one thread per value row)
  if (tid < kD) {
    double t = 0.0;
    for (int g = 0; g < 16; ++g) t += L.part.upart[g * kD + tid];
    const float uu = (float)((double)L.rf[tid] * t);
    L.w[tid] = b[u] * (L.v[tid] - uu);
  }
  __syncthreads();

  // 4. rank-one update and readout partials
  float km[8], qm[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    km[m] = L.k[p0 + m];
    qm[m] = L.q[p0 + m];
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int i = rg + 16 * rr;
    const float wi = L.w[i];
    float oacc = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      s[rr][m] = fmaf(wi, km[m], s[rr][m]);
      oacc = fmaf(s[rr][m], qm[m], oacc);
    }
    L.part.f.opart[(w * 4 + jg) * kD + i] = oacc;
  }

  // 5. refit scales (writes R, c) and collect the readout
  refit_tail(s, w, rg, jg, sg.bits, L.tail, Rs + uo, Cs + uo);
  if (tid >= kD) {
    const int i = tid - kD;
    float os = 0.0f;
    for (int g = 0; g < 16; ++g) os += L.part.f.opart[g * kD + i];
    o[uo + i] = os;
  }
  __syncthreads();

  // 6. requantize and store in place
  const float qmax = (float)((1 << (sg.bits - 1)) - 1);
  float M[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) M[rr] = qmax * L.tail.invc[rg + 16 * rr];
  requant_dispatch(sg.bits, seg, rg, jg, s, M);
}

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
                     p.req_bytes, S, packed, rs, cs);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Pool& p, const uint8_t* packed, const float* rs,
                             const float* cs, float* S, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequantize, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                     p.req_bytes, packed, rs, cs, S);
  return hipGetLastError();
}

hipError_t launch_step(const Pool& p, int gate, uint8_t* packed, float* rs, float* cs,
                       const float* q, const float* k, const float* v, const float* a,
                       const float* b, float* o, hipStream_t s) {
  if (p.n_unit == 0) return hipSuccess;
  if (gate == GDN)
    hipLaunchKernelGGL(k_step<GDN>, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                       p.req_bytes, packed, rs, cs, q, k, v, a, b, o);
  else
    hipLaunchKernelGGL(k_step<KDA>, dim3(p.n_unit), dim3(kThreads), 0, s, p.meta, p.n_head,
                       p.req_bytes, packed, rs, cs, q, k, v, a, b, o);
  return hipGetLastError();
}

}  // namespace qdr
