// qdr_internal.h -- shared between the C-ABI host layer and the gfx950 kernels of libqdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qdr {

constexpr int kD = 128;          // dk = dv = 128 (STEPQuant page, Fig. 5 / Figure B2)
constexpr int kSeg = 32;         // key positions per segment (one width per segment)
constexpr int kThreads = 256;    // one work-group of 4 wave64 per (request, head) unit
constexpr uint32_t kMetaMagic = 0x31524451u;  // "QDR1"
constexpr int kWindowMax = 256;  // largest window (tokens) of qdr_decode_window

// Device metadata table: a 64-byte header, then one MetaHead per head.
struct MetaHeader {
  uint32_t magic;
  uint32_t n_head;
  uint32_t dk, dv;
  uint32_t gate;
  uint32_t req_bytes;
  uint32_t window;
  uint32_t uniform;     // 1 if every head has a single code width
  uint32_t n_class[3];  // uniform heads of width 8, 6, 4
  uint32_t reserved[5];
};
static_assert(sizeof(MetaHeader) == 64, "meta header size");

struct MetaHead {
  uint32_t tile_off;    // byte offset of the head's tile inside a request
  uint32_t tile_bytes;  // 16 * sum_j bits_j
  uint8_t seg_bits[4];  // width of physical positions 32s..32s+31
  uint32_t identity;    // 1 if the physical order is the logical order
  uint8_t perm[kD];     // perm[p] = logical key channel at physical position p
  uint8_t iperm[kD];    // iperm[j] = physical position of logical key channel j
};
static_assert(sizeof(MetaHead) == 272, "meta head size");

__host__ __device__ inline const MetaHead* meta_heads(const void* meta) {
  return reinterpret_cast<const MetaHead*>(static_cast<const uint8_t*>(meta) + sizeof(MetaHeader));
}

// After the head records: uint16 head indices ordered by width (8, 6, 4), ties by index
// (meaningful when every head has a single width).
__host__ __device__ inline const uint16_t* meta_order(const void* meta, int n_head) {
  return reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(meta) + sizeof(MetaHeader) +
                                           (size_t)n_head * sizeof(MetaHead));
}

inline size_t meta_bytes(int n_head) {
  return sizeof(MetaHeader) + (size_t)n_head * sizeof(MetaHead) +
         (((size_t)n_head * 2 + 15) & ~(size_t)15);
}

// Bytes of one window-buffer slot set per unit: W slots of (kappa[128], delta[128]) fp32
// plus the running cumulative gate g[128] and the buffered keys' decay since their base
// h[128], fp32.
__host__ __device__ inline size_t window_unit_bytes(int W) { return (size_t)W * 2 * kD * 4 + (size_t)2 * kD * 4; }

struct Pool {
  const void* meta;
  int n_head;
  int n_unit;
  uint32_t req_bytes;
  int uniform;      // every head has a single code width
  int n_class[3];   // heads of width 8, 6, 4 (uniform case)
  int rule;         // scale rule (QDR_RULE_*)
};

// Launchers (kernels.hip). All enqueue on `stream` and return hipGetLastError().
hipError_t launch_init(const Pool& p, uint8_t* packed, float* rs, float* cs, hipStream_t s);
hipError_t launch_quantize(const Pool& p, const float* S, uint8_t* packed, float* rs, float* cs,
                           hipStream_t s);
hipError_t launch_dequantize(const Pool& p, const uint8_t* packed, const float* rs,
                             const float* cs, float* S, hipStream_t s);
hipError_t launch_step(const Pool& p, int gate, uint8_t* packed, float* rs, float* cs,
                       const float* q, const float* k, const float* v, const float* a,
                       const float* b, float* o, hipStream_t s);
// One window token (and, at t = W-1, the fold and requantization).
hipError_t launch_window(const Pool& p, int gate, int W, int t, uint8_t* packed, float* rs,
                         float* cs, uint8_t* buf, const float* q, const float* k, const float* v,
                         const float* a, const float* b, float* o, int m, uint16_t* tok_idx,
                         float* tok_val, hipStream_t s);

// T tokens of every unit in one call; token-major inputs [T][unit][...].
// m > 0: compensator tokens tok_idx / tok_val [n_unit][m] (read at the start, rewritten
// at the end); S_in (with T = 0): quantize the given fp32 state instead of a chunk.
hipError_t launch_chunk(const Pool& p, int gate, int T, uint8_t* packed, float* rs, float* cs,
                        const float* q, const float* k, const float* v, const float* a,
                        const float* b, float* o, int m, uint16_t* tok_idx, float* tok_val,
                        const float* S_in, hipStream_t s);
// S [n_unit][128][128] += the compensator tokens
hipError_t launch_comp_add(int n_unit, int m, const uint16_t* tok_idx, const float* tok_val,
                           float* S, hipStream_t s);
constexpr int kCompMax = 64;

// DAMP-style storage variant (qdr_damp.hip)
constexpr int kDampHalf = 16;  // key channels per head kept in binary16
struct DampPool {
  const uint8_t* perm;  // device [n_head][128]: physical position -> logical channel
  int n_head, n_unit, gate;
  int ident;  // every head selects channels 0..15 (then perm is the identity)
};
enum { kDampInit = 0, kDampQuantize = 1, kDampStep = 2, kDampDequantize = 3 };
hipError_t launch_damp(int op, const DampPool& p, uint16_t* half, int8_t* codes, float* R,
                       const float* q, const float* k, const float* v, const float* a,
                       const float* b, float* o, const float* S, float* Sout, uint64_t seed,
                       uint64_t step, hipStream_t s);

// Correctly rounded divisions shared by the kernels.
// 1/x, correctly rounded (the IEEE division): for x in [2^-126, 2^126) the hardware
// reciprocal followed by one Newton step r = y + y(1 - xy) (two fmas) is exactly that --
// checked on the GPU against the division for every fp32 pattern of that range; for
// subnormal x, or x whose reciprocal is subnormal, the division itself runs (such
// scales are rare, so the lanes almost never take that branch).
__device__ __forceinline__ float recip_rn(float x) {
  const float y = __builtin_amdgcn_rcpf(x);
  const float e = fmaf(-x, y, 1.0f);
  float r = fmaf(e, y, y);
  if (__builtin_amdgcn_ballot_w64(!(x >= 0x1p-126f && x < 0x1p126f))) {
    // a branch the wave skips when no lane needs it (the empty volatile asm keeps the
    // compiler from evaluating the division unconditionally)
    float xx = x;
    asm volatile("" : "+v"(xx));
    if (!(xx >= 0x1p-126f && xx < 0x1p126f)) r = 1.0f / xx;
  }
  return r;
}

// a / Qmax for Qmax = 2^(b-1) - 1 (b in {4, 6, 8}), correctly rounded: the product with
// fl(1/Qmax) and one remainder correction, q = q0 + fl(1/Qmax)(a - q0 Qmax) (two fmas,
// the remainder exact) -- equal to the IEEE division for every positive fp32 a and each
// of the three Qmax (checked on the GPU over every fp32 pattern).
__device__ __forceinline__ float div_qmax(float a, int b) {
  const float q = b == 8 ? 127.0f : (b == 6 ? 31.0f : 7.0f);
  const float iq = b == 8 ? 1.0f / 127.0f : (b == 6 ? 1.0f / 31.0f : 1.0f / 7.0f);
  const float q0 = a * iq;
  const float r = fmaf(-q0, q, a);
  return fmaf(r, iq, q0);
}

}  // namespace qdr
