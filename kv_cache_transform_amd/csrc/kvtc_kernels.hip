// HIP kernels of KV-cache transform coding for gfx950 (MI355X).
//
// Method: "KV Cache Transform Coding for Compact Storage in LLM Inference"
// (gist.science, 2511.01815), section 2B (compression: subtract the mean,
// multiply by V, quantize with the DP widths, pack) and section 2C
// (decompression: dequantize, multiply by V^T, add the mean, layer by layer).
//
// Every launch covers a batch of jobs (tensors). The grid is a flat list of
// logical tiles; tiles of one job are consecutive and the blockIdx -> tile map
// sends consecutive tiles to the same XCD, so one tensor's basis stays in one
// XCD's L2.
//
// Encode tile (256 threads, 128 tokens): the four waves each own 32 tokens.
// The projection runs on v_mfma_f32_32x32x16_bf16 in transposed form,
// D[component][token] = sum_f V'^T[component][f] * x'[token][f]: the basis
// K-slice is staged in LDS and shared by the waves, the centred tokens
// x' = bf16_rne(fp32(x) - mu) are formed in registers straight from global
// memory. In the accumulator layout a lane owns one token and half of every
// group's components, so the per-(token, group) min/max needs one cross-lane
// exchange (lane ^ 32), quantization is lane-local, and a second exchange
// gives each lane G/2 consecutive codes that it packs into one or two 64-bit
// words. Records are assembled in LDS and leave in 16-byte stores.
//
// Decode tile (256 threads, 128 tokens): records are staged into LDS with
// 16-byte loads; each lane rebuilds its token's dequantized coefficients
// c_hat = shift + q * fp32(scale / k) for the 8 components it feeds to the
// MFMA, scaled by a per-token power of two into fp16 (the fp16 operand keeps
// 11 significant bits; the scale makes the range irrelevant), then runs
// D[feature][token] = sum_j V'[feature][j] * c_hat[token][j] on
// v_mfma_f32_32x32x16_f16 per 32-feature block and writes S_t * D + mu.
#include <hip/hip_runtime.h>

#include "kvtc_internal.h"

namespace kvtc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// ------------------------------------------------------------- helpers ---

__device__ __forceinline__ uint32_t logical_tile() {
  const uint32_t n8 = gridDim.x >> 3;      // grid is a multiple of 8
  return (blockIdx.x & 7u) * n8 + (blockIdx.x >> 3);
}

__device__ __forceinline__ int find_job(const LaunchArgs& a, uint32_t tile) {
  int j = 0;
  for (int i = 1; i < a.n_jobs; ++i)
    if (a.jobs[i].tile_begin <= tile) j = i;
  return j;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> packed bf16 / fp16, round to nearest even (v_cvt_pk_*_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// 8 bytes from any LDS byte address: three aligned dword reads and two
// byte-aligns (the buffer is padded so the last read stays inside it).
__device__ __forceinline__ uint64_t lds_u64(const uint8_t* p) {
  const uintptr_t a = (uintptr_t)p;
  const uint32_t* b = (const uint32_t*)(a & ~(uintptr_t)3);
  const uint32_t sh = (uint32_t)(a & 3u);
  const uint32_t w0 = b[0], w1 = b[1], w2 = b[2];
  const uint32_t lo = __builtin_amdgcn_alignbyte(w1, w0, sh);
  const uint32_t hi = __builtin_amdgcn_alignbyte(w2, w1, sh);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ size_t record_base(const JobDesc& jd, int F, int esz) {
  return (size_t)kHeaderBytes + (size_t)(jd.s1 + jd.w1) * F * esz;
}

__device__ void write_header(const LaunchArgs& a, const JobDesc& jd, const DevSlot& sl) {
  uint32_t h[16];
  h[0] = 0x4354564Bu;  // "KVTC"
  h[1] = (uint32_t)kFormatVersion | ((uint32_t)a.dtype << 16) | ((uint32_t)jd.kind << 24);
  h[2] = (uint32_t)jd.layer;
  h[3] = jd.T;
  h[4] = (uint32_t)a.F;
  h[5] = jd.s1;
  h[6] = jd.w1;
  h[7] = jd.tc;
  h[8] = (uint32_t)sl.G | ((uint32_t)sl.n_act << 16);
  h[9] = (uint32_t)sl.record_bytes;
  h[10] = (uint32_t)sl.slot_id;
  h[11] = (uint32_t)(sl.slot_id >> 32);
  h[12] = h[13] = h[14] = h[15] = 0;
  uint4* d = (uint4*)jd.dst;
  for (int i = 0; i < 4; ++i) d[i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
}

// Returns KVTC_OK or the status a stream with this header earns.
__device__ int check_header(const LaunchArgs& a, const JobDesc& jd, const DevSlot& sl) {
  const uint32_t* h = (const uint32_t*)jd.src;
  if (h[0] != 0x4354564Bu || (h[1] & 0xFFFFu) != kFormatVersion) return KVTC_E_CORRUPT;
  const uint32_t want1 = (uint32_t)kFormatVersion | ((uint32_t)a.dtype << 16) | ((uint32_t)jd.kind << 24);
  if (h[1] != want1 || h[2] != (uint32_t)jd.layer || h[3] != jd.T || h[4] != (uint32_t)a.F ||
      h[5] != jd.s1 || h[6] != jd.w1 || h[7] != jd.tc ||
      h[8] != ((uint32_t)sl.G | ((uint32_t)sl.n_act << 16)) || h[9] != (uint32_t)sl.record_bytes ||
      h[10] != (uint32_t)sl.slot_id || h[11] != (uint32_t)(sl.slot_id >> 32))
    return KVTC_E_MISMATCH;
  return KVTC_OK;
}

__device__ __forceinline__ void set_status(const LaunchArgs& a, int j, int st) {
  atomicMax(&a.status[j], ((unsigned long long)a.epoch << 32) | (unsigned long long)status_rank(st));
}

// Rank an earlier launch on this workspace (stage 1) recorded for job j;
// results this launch wrote itself do not count.
__device__ __forceinline__ int prior_rank(const LaunchArgs& a, int j) {
  const unsigned long long w = a.status[j];
  return (uint32_t)(w >> 32) == a.epoch ? 0 : (int)(w & 0xFFull);
}

// Physical output row of token t (contiguous or through the block table);
// -1 if the block table entry is out of range.
__device__ __forceinline__ long out_row(const JobDesc& jd, uint32_t t) {
  if (!jd.block_table) return (long)t;
  const int blk = jd.block_table[t / (uint32_t)jd.block_size];
  if (blk < 0 || blk >= jd.n_blocks) return -1;
  return (long)blk * jd.block_size + (long)(t % (uint32_t)jd.block_size);
}

// Encode: copy passthrough rows [p*kPassRows, ...) of the stream's row list
// (rows [0, s') then [T - w', T)) from the KV tensor into the stream.
__device__ void encode_passthrough(const JobDesc& jd, uint32_t p, size_t row_bytes) {
  const uint32_t n_rows = jd.s1 + jd.w1;
  const uint32_t r0 = p * kPassRows;
  const uint32_t r1 = min(n_rows, r0 + kPassRows);
  const size_t vec_per_row = row_bytes / 16;
  const size_t total = (size_t)(r1 - r0) * vec_per_row;
  for (size_t i = threadIdx.x; i < total; i += kThreads) {
    const uint32_t r = r0 + (uint32_t)(i / vec_per_row);
    const size_t c = i % vec_per_row;
    const uint32_t src_row = r < jd.s1 ? r : jd.T - jd.w1 + (r - jd.s1);
    const uint4 v = ((const uint4*)((const uint8_t*)jd.src + (size_t)src_row * row_bytes))[c];
    ((uint4*)((uint8_t*)jd.dst + kHeaderBytes + (size_t)r * row_bytes))[c] = v;
  }
}

// Decode: copy passthrough rows from the stream to the output, converting
// the element type if needed. Returns false if a block table entry was bad.
__device__ bool decode_passthrough(const LaunchArgs& a, const JobDesc& jd, uint32_t p) {
  const int F = a.F;
  const uint32_t n_rows = jd.s1 + jd.w1;
  const uint32_t r0 = p * kPassRows;
  const uint32_t r1 = min(n_rows, r0 + kPassRows);
  const int in_esz = a.dtype == KVTC_F32 ? 4 : 2;
  const int out_esz = a.out_dtype == KVTC_F32 ? 4 : 2;
  const uint8_t* src = (const uint8_t*)jd.src + kHeaderBytes;
  bool ok = true;
  if (a.dtype == a.out_dtype) {
    const size_t vec_per_row = (size_t)F * in_esz / 16;
    const size_t total = (size_t)(r1 - r0) * vec_per_row;
    for (size_t i = threadIdx.x; i < total; i += kThreads) {
      const uint32_t r = r0 + (uint32_t)(i / vec_per_row);
      const size_t c = i % vec_per_row;
      const uint32_t t = r < jd.s1 ? r : jd.T - jd.w1 + (r - jd.s1);
      const long orow = out_row(jd, t);
      if (orow < 0) { ok = false; continue; }
      const uint4 v = ((const uint4*)(src + (size_t)r * F * in_esz))[c];
      ((uint4*)((uint8_t*)jd.dst + (size_t)orow * F * out_esz))[c] = v;
    }
  } else {
    const size_t total = (size_t)(r1 - r0) * F;
    for (size_t i = threadIdx.x; i < total; i += kThreads) {
      const uint32_t r = r0 + (uint32_t)(i / F);
      const int c = (int)(i % F);
      const uint32_t t = r < jd.s1 ? r : jd.T - jd.w1 + (r - jd.s1);
      const long orow = out_row(jd, t);
      if (orow < 0) { ok = false; continue; }
      if (a.dtype == KVTC_BF16) {  // bf16 -> f32, exact
        const uint16_t b = ((const uint16_t*)(src + (size_t)r * F * 2))[c];
        ((float*)jd.dst)[(size_t)orow * F + c] = bf16_to_f32(b);
      } else {                     // f32 -> bf16, nearest even
        const float f = ((const float*)(src + (size_t)r * F * 4))[c];
        ((uint16_t*)jd.dst)[(size_t)orow * F + c] = (uint16_t)bf16_bits_rne(f);
      }
    }
  }
  return ok;
}

// Copy n bytes from 16-byte aligned global memory into LDS (cooperative).
__device__ void stage_to_lds(uint8_t* lds, const uint8_t* g, size_t n) {
  const size_t nv = n / 16;
  for (size_t i = threadIdx.x; i < nv; i += kThreads) ((uint4*)lds)[i] = ((const uint4*)g)[i];
  for (size_t i = nv * 16 + threadIdx.x; i < n; i += kThreads) lds[i] = g[i];
}

// Copy n bytes from LDS to 16-byte aligned global memory (cooperative).
__device__ void lds_to_global(uint8_t* g, const uint8_t* lds, size_t n) {
  const size_t nv = n / 16;
  for (size_t i = threadIdx.x; i < nv; i += kThreads) ((uint4*)g)[i] = ((const uint4*)lds)[i];
  for (size_t i = nv * 16 + threadIdx.x; i < n; i += kThreads) g[i] = lds[i];
}

// Pack n codes of width w (LSB first) into a 64-bit word (n * w <= 64).
__device__ __forceinline__ uint64_t pack_codes(const uint32_t* q, int n, int w) {
  uint64_t bits = 0;
  for (int j = 0; j < n; ++j) bits |= (uint64_t)q[j] << (j * w);
  return bits;
}

// Store the low n bytes of v at an arbitrary LDS byte address.
__device__ __forceinline__ void lds_store_bytes(uint8_t* p, uint64_t v, int n) {
  for (int i = 0; i < n; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

// Load n (<= 8) bytes from an arbitrary LDS/global byte address.
__device__ __forceinline__ uint64_t load_bytes(const uint8_t* p, int n) {
  uint64_t v = 0;
  for (int i = 0; i < n; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

// Write the G/2 codes a lane holds for active group `a` (half h) and, for
// h == 0, the group's (shift, scale), into the token's record.
template <int G>
__device__ __forceinline__ void put_group(uint8_t* rec, const DevSlot& sl, int a, int h,
                                          const uint32_t* codes, float shift, float scale) {
  const int w = sl.width[a];
  const int half_bytes = (G / 2) * w / 8;
  uint8_t* p = rec + sl.chunk_off[a] + h * half_bytes;
  if (G == 16) {
    lds_store_bytes(p, pack_codes(codes, 8, w), w);
  } else {
    lds_store_bytes(p, pack_codes(codes, 8, w), w);
    lds_store_bytes(p + w, pack_codes(codes + 8, 8, w), w);
  }
  if (h == 0) {
    const uint32_t s = __float_as_uint(shift), c = __float_as_uint(scale);
    lds_store_bytes(rec + 8 * a, (uint64_t)s | ((uint64_t)c << 32), 8);
  }
}

// The 8 codes of components [o, o + 8) of active group a from a record:
// one byte per code in a 64-bit word.
__device__ __forceinline__ uint64_t get_codes8(const uint8_t* rec, const DevSlot& sl, int a, int o) {
  const int w = sl.width[a];
  const uint64_t bits = lds_u64(rec + sl.chunk_off[a] + (o * w) / 8);
  const uint64_t mask = (1ull << w) - 1ull;
  uint64_t out = 0;
  for (int j = 0; j < 8; ++j) out |= ((bits >> (j * w)) & mask) << (8 * j);
  return out;
}

// --------------------------------------------------------------- encode ---

template <int NB, int G, bool F32IN>
__global__ __launch_bounds__(kThreads) void encode_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const int j = find_job(a, tile);
  const JobDesc& jd = a.jobs[j];
  const DevSlot& sl = ((const DevSlot*)a.state)[jd.slot];
  const uint32_t lt = tile - jd.tile_begin;
  const int F = a.F;
  constexpr int esz = F32IN ? 4 : 2;
  const size_t row_bytes = (size_t)F * esz;
  if (lt == 0 && threadIdx.x == 0) {
    write_header(a, jd, sl);
    set_status(a, jd.status_idx, KVTC_OK);
  }
  if (lt >= jd.n_ctiles) {
    encode_passthrough(jd, lt - jd.n_ctiles, row_bytes);
    return;
  }
  const uint32_t t0 = lt * kEncTile;
  const uint32_t n = min((uint32_t)kEncTile, jd.tc - t0);
  const int rb = sl.record_bytes;
  if (sl.r_eff == 0) return;  // zero-width records: nothing to write

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);            // token within the tile
  const bool tok_ok = (uint32_t)tl < n;
  const uint8_t* xrow = (const uint8_t*)jd.src + (size_t)(jd.s1 + t0 + (tok_ok ? tl : 0)) * row_bytes;
  const uint16_t* venc = (const uint16_t*)(a.state + sl.venc_off);

  // LDS: two basis K-slices [32 * NB][kEncRowPad] bf16, then the mean (F fp32).
  constexpr int slice_elems = 32 * NB * kEncRowPad;
  uint16_t* const vbase = (uint16_t*)smem;
  float* mu_l = (float*)(smem + (size_t)4 * slice_elems);
  {
    const float4* mu = (const float4*)(a.state + sl.mu_off);
    for (int i = threadIdx.x; i < F / 4; i += kThreads) ((float4*)mu_l)[i] = mu[i];
  }
  // Slice copy: a slice holds 32 * NB rows of kEncKS features, 32 * NB * 8
  // vectors of 16 bytes, so thread t moves vectors t + q * kThreads, q < NB,
  // with no predicate. Rows >= r_enc (zero in the device state when r_enc
  // < 32 * NB, clamped re-reads otherwise) are never read by the MFMA loop.
  typedef uint32_t vregs_t __attribute__((ext_vector_type(4 * NB)));
  vregs_t vreg;
  const int vlast = sl.r_enc * (kEncKS / 8) - 1;
#define KVTC_LOAD_SLICE(K0)                                                          \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                   \
    const int idx = min((int)threadIdx.x + q * kThreads, vlast);                     \
    const uint4 v = *(const uint4*)(venc + (size_t)(idx / (kEncKS / 8)) * F + (K0) + \
                                    (idx % (kEncKS / 8)) * 8);                       \
    vreg[4 * q] = v.x;                                                               \
    vreg[4 * q + 1] = v.y;                                                           \
    vreg[4 * q + 2] = v.z;                                                           \
    vreg[4 * q + 3] = v.w;                                                           \
  }
#define KVTC_STORE_SLICE(BUF)                                                        \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                   \
    const int idx = (int)threadIdx.x + q * kThreads;                                 \
    *(uint4*)((BUF) + (idx / (kEncKS / 8)) * kEncRowPad + (idx % (kEncKS / 8)) * 8) = \
        make_uint4(vreg[4 * q], vreg[4 * q + 1], vreg[4 * q + 2], vreg[4 * q + 3]);  \
  }
  // Token fragments of one slice: K step s reads features k0 + 16s + 8h .. +8.
  constexpr int XV = F32IN ? 2 : 1;                  // 16-byte vectors per K step
  uint4 xr[4 * XV], xn[4 * XV];
  auto load_x = [&](int k0, uint4* dst) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int v = 0; v < XV; ++v)
        dst[s * XV + v] = *(const uint4*)(xrow + (size_t)(k0 + 16 * s + 8 * h) * esz + 16 * v);
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;

  KVTC_LOAD_SLICE(0)
  load_x(0, xr);
  KVTC_STORE_SLICE(vbase)
  __syncthreads();
  int it = 0;
  for (int k0 = 0; k0 < F; k0 += kEncKS, ++it) {
    const bool more = k0 + kEncKS < F;
    if (more) {
      KVTC_LOAD_SLICE(k0 + kEncKS)
      load_x(k0 + kEncKS, xn);
    }
    const uint16_t* vs = vbase + (it & 1) * slice_elems;
#pragma unroll
    for (int s = 0; s < kEncKS / 16; ++s) {
      const int f = k0 + 16 * s + 8 * h;
      // Centred token operand: x' = bf16_rne(fp32(x) - mu).
      float xv[8];
      if (!F32IN) {
        const uint4 raw = xr[s];
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = bf16_to_f32(w4[e] & 0xFFFFu);
          xv[2 * e + 1] = bf16_to_f32(w4[e] >> 16);
        }
      } else {
        const uint4 lo = xr[2 * s], hi = xr[2 * s + 1];
        xv[0] = __uint_as_float(lo.x); xv[1] = __uint_as_float(lo.y);
        xv[2] = __uint_as_float(lo.z); xv[3] = __uint_as_float(lo.w);
        xv[4] = __uint_as_float(hi.x); xv[5] = __uint_as_float(hi.y);
        xv[6] = __uint_as_float(hi.z); xv[7] = __uint_as_float(hi.w);
      }
      const float4 m0 = *(const float4*)(mu_l + f);
      const float4 m1 = *(const float4*)(mu_l + f + 4);
      const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(xv[2 * e] - mv[2 * e], xv[2 * e + 1] - mv[2 * e + 1]);
      const bf16x8 bx = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 av = *(const uint4*)(vs + (b * 32 + (lane & 31)) * kEncRowPad + 16 * s + 8 * h);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bx,
                                                         acc[b], 0, 0, 0);
      }
    }
    if (more) {
      KVTC_STORE_SLICE(vbase + ((it + 1) & 1) * slice_elems)
#pragma unroll
      for (int v = 0; v < 4 * XV; ++v) xr[v] = xn[v];
    }
    __syncthreads();
  }
#undef KVTC_LOAD_SLICE
#undef KVTC_STORE_SLICE

  // Quantize and pack. acc[b][i] holds component 32b + 8(i/4) + 4h + i%4 of
  // token tl; a group of G components is the item range
  // [(G/2) * sg, (G/2) * (sg + 1)) of block b with sg = a % (32/G).
  uint8_t* rec = smem + (size_t)tl * rb;
  constexpr int SUB = 32 / G;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int sg = 0; sg < SUB; ++sg) {
      const int ag = b * SUB + sg;
      if (ag < sl.n_act) {
        float v[G / 2];
#pragma unroll
        for (int i = 0; i < G / 2; ++i) v[i] = acc[b][(G / 2) * sg + i];
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < G / 2; ++i) {
          mn = fminf(mn, v[i]);
          mx = fmaxf(mx, v[i]);
        }
        mn = fminf(mn, __shfl_xor(mn, 32));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const int w = sl.width[ag];
        const float k = (float)((1 << w) - 1);
        const float scale = mx - mn;
        const float inv = scale > 0.f ? k / scale : 0.f;
        uint32_t quad[G / 8];
#pragma unroll
        for (int m = 0; m < G / 8; ++m) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = v[4 * m + e] - mn;
            const float u = d * inv;
            const float r = fminf(fmaxf(__builtin_rintf(u), 0.f), k);
            word |= (uint32_t)r << (8 * e);
          }
          quad[m] = word;
        }
        // Lane h holds the group's component quads 2m + h; gather quads
        // [h * G/8, (h + 1) * G/8) so each lane packs G/2 consecutive codes.
        uint32_t recv[G / 8];
#pragma unroll
        for (int m = 0; m < G / 8; ++m) recv[m] = __shfl_xor(quad[m], 32);
        uint32_t codes[G / 2];
#pragma unroll
        for (int m = 0; m < G / 8; ++m) {
          const int q0 = m, q1 = G / 8 + m;  // target quad for h = 0 / h = 1
          const uint32_t c0 = (q0 % 2 == 0) ? quad[q0 / 2] : recv[q0 / 2];
          const uint32_t c1 = (q1 % 2 == 1) ? quad[q1 / 2] : recv[q1 / 2];
          const uint32_t word = h ? c1 : c0;
#pragma unroll
          for (int e = 0; e < 4; ++e) codes[4 * m + e] = (word >> (8 * e)) & 0xFFu;
        }
        if (tok_ok) put_group<G>(rec, sl, ag, h, codes, mn, scale);
      }
    }
  }
  __syncthreads();
  uint8_t* dst = (uint8_t*)jd.dst + record_base(jd, F, esz) + (size_t)t0 * rb;
  lds_to_global(dst, smem, (size_t)n * rb);
}

// --------------------------------------------------------------- decode ---

// Per-token power-of-two scale: S = 2^(e - 14) where 2^e <= max |c_hat| over
// the token's groups < 2^(e+1), so the fp16 operand peaks in [2^14, 2^15).
__device__ __forceinline__ void token_scale(float m, float& S, float& Sinv) {
  int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
  if (m == 0.f) e = 14;
  e = max(min(e, 100), -100);
  S = __uint_as_float((uint32_t)(127 + e - 14) << 23);
  Sinv = __uint_as_float((uint32_t)(127 + 14 - e) << 23);
}

// Dequantize 8 codes (one byte each in codes8) of a group of width w and
// scale them by Sinv into packed fp16: c_hat = fma(q, fp32(scale / k), shift).
__device__ __forceinline__ uint4 make_frag(uint64_t codes8, float shift, float scale, int w,
                                           float Sinv) {
  const float k = (float)((1 << w) - 1);
  const float step = scale / k;
  uint32_t pk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float q0 = (float)((codes8 >> (16 * j)) & 0xFFu);
    const float q1 = (float)((codes8 >> (16 * j + 8)) & 0xFFu);
    pk[j] = pack_f16x2(__builtin_fmaf(q0, step, shift) * Sinv, __builtin_fmaf(q1, step, shift) * Sinv);
  }
  return make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// 8 bytes from global memory at any byte address p inside [., end): three
// aligned dword loads and two byte-aligns, or byte loads near the end so that
// nothing past `end` is touched.
__device__ __forceinline__ uint64_t gl_u64(const uint8_t* p, const uint8_t* end) {
  const uintptr_t a = (uintptr_t)p;
  if (p + 12 <= end) {
    const uint32_t* b = (const uint32_t*)(a & ~(uintptr_t)3);
    const uint32_t sh = (uint32_t)(a & 3u);
    const uint32_t w0 = b[0], w1 = b[1], w2 = b[2];
    return (uint64_t)__builtin_amdgcn_alignbyte(w1, w0, sh) |
           ((uint64_t)__builtin_amdgcn_alignbyte(w2, w1, sh) << 32);
  }
  uint64_t v = 0;
  for (int i = 0; i < 8 && p + i < end; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

// Unpack the 8 codes of components [o, o + 8) of active group a from packed
// bits (LSB first), one byte per code.
__device__ __forceinline__ uint64_t spread_codes8(uint64_t bits, int w) {
  const uint64_t mask = (1ull << w) - 1ull;
  uint64_t out = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) out |= ((bits >> (j * w)) & mask) << (8 * j);
  return out;
}

constexpr int kChatPad = 16;  // bytes of padding per LDS c_hat row

// LDS bytes of a decode tile: the c_hat rows (reused for output staging),
// the per-token scale words and the mean.
__host__ __device__ inline size_t dec_lds_bytes(int r_dec, int F) {
  const size_t chat = (size_t)kDecTile * (2 * r_dec + kChatPad);
  const size_t outs = (size_t)4 * 32 * kOutRow;
  return align_up(chat > outs ? chat : outs, 16) + 4 * kDecTile + 4 * (size_t)F;
}

// Compressed rows of one tile (128 tokens; wave w owns tokens 32w..32w+31).
//  1. the mean goes to LDS; per token the scale S_t is the power of two
//     above max |c_hat| (LDS atomicMax over its groups);
//  2. cooperative dequantization: one thread per (token, 8 components)
//     writes c_hat / S_t as fp16 into LDS; codes come straight from the
//     stream's records (fused) or the staging buffer (two-stage);
//  3. each lane loads its token's KS B fragments from LDS;
//  4. per 32-feature block, KS MFMAs D[feature][token] = V' c_hat^T with the
//     basis fragments of the next block already in flight (two register
//     sets, no copies), then S_t * D + mu, staged through LDS so that stores
//     are 16-byte lanes over 128-byte row segments.
template <int KS, bool OUT32, bool STAGED>
__device__ void restore_tile(const LaunchArgs& a, const JobDesc& jd, const DevSlot& sl,
                             uint8_t* smem, uint32_t t0, uint32_t n, int* bad) {
  const int F = a.F;
  const int r_eff = sl.r_eff, r_dec = sl.r_dec, n_act = sl.n_act, G = sl.G;
  const int rb = sl.record_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);
  const size_t chat_stride = 2 * (size_t)r_dec + kChatPad;
  const size_t chat_bytes = align_up(max((size_t)kDecTile * chat_stride, (size_t)4 * 32 * kOutRow), 16);
  uint8_t* chat = smem;
  uint32_t* sbits = (uint32_t*)(smem + chat_bytes);
  float* mu_l = (float*)(sbits + kDecTile);
  const float4* mu_g = (const float4*)(a.state + sl.mu_off);
  for (int i = threadIdx.x; i < F / 4; i += kThreads) ((float4*)mu_l)[i] = mu_g[i];
  if (threadIdx.x < kDecTile) sbits[threadIdx.x] = 0u;

  // Code sources.
  const int esz = a.dtype == KVTC_F32 ? 4 : 2;
  const uint8_t* recs = nullptr;
  const uint8_t* rec_end = nullptr;
  const uint8_t* scodes = nullptr;
  const float2* sss = nullptr;
  if (STAGED) {
    const uint8_t* st = (const uint8_t*)jd.staging;
    scodes = st + (size_t)t0 * r_eff;
    sss = (const float2*)(st + align_up((size_t)jd.tc * r_eff, kAlign)) + (size_t)t0 * n_act;
  } else {
    const uint8_t* base = (const uint8_t*)jd.src + record_base(jd, F, esz);
    recs = base + (size_t)t0 * rb;
    rec_end = base + (size_t)jd.tc * rb;
  }
  auto ss_of = [&](int t, int g) -> float2 {
    if (STAGED) return sss[(size_t)t * n_act + g];
    const uint64_t raw = gl_u64(recs + (size_t)t * rb + 8 * g, rec_end);
    return make_float2(__uint_as_float((uint32_t)raw), __uint_as_float((uint32_t)(raw >> 32)));
  };
  __syncthreads();
  // 1. per-token scales (max over groups; non-negative floats order as ints)
  for (int i = threadIdx.x; i < (int)n * n_act; i += kThreads) {
    const int t = i / n_act, g = i - t * n_act;
    const float2 p = ss_of(t, g);
    const float m = fmaxf(fabsf(p.x), fabsf(p.x + p.y));
    atomicMax(&sbits[t], __float_as_uint(m));
  }
  __syncthreads();
  // 2. c_hat / S_t in fp16, 8 components per item
  const int c8n = r_dec / 8;
  for (int i = threadIdx.x; i < (int)n * c8n; i += kThreads) {
    const int t = i / c8n, c = (i - t * c8n) * 8;
    uint4 frag = make_uint4(0u, 0u, 0u, 0u);
    if (c < r_eff) {
      float S, Sinv;
      token_scale(__uint_as_float(sbits[t]), S, Sinv);
      const int ag = c / G, o = c - ag * G;
      const int w = sl.width[ag];
      uint64_t codes8;
      if (STAGED)
        codes8 = *(const uint64_t*)(scodes + (size_t)t * r_eff + c);
      else
        codes8 = spread_codes8(gl_u64(recs + (size_t)t * rb + sl.chunk_off[ag] + (o * w) / 8, rec_end), w);
      const float2 p = ss_of(t, ag);
      frag = make_frag(codes8, p.x, p.y, w, Sinv);
    }
    *(uint4*)(chat + (size_t)t * chat_stride + 2 * c) = frag;
  }
  __syncthreads();
  // 3. this lane's B fragments and token scale
  uint4 bfr[KS > 0 ? KS : 1];
#pragma unroll
  for (int s = 0; s < KS; ++s) bfr[s] = *(const uint4*)(chat + (size_t)tl * chat_stride + 2 * (16 * s + 8 * h));
  float S, Sinv;
  token_scale(__uint_as_float(sbits[tl]), S, Sinv);
  __syncthreads();  // the c_hat region becomes the output staging area

  // Store rows of this lane: row r = 8 * it + lane / 8 of the wave's 32
  // tokens, 16 bytes at column (lane % 8) * 16 of a 128-byte segment.
  constexpr int OSZ = OUT32 ? 4 : 2;
  constexpr int FPG = 128 / (32 * OSZ);               // feature blocks per 128-byte segment
  const int c16 = lane & 7;
  long orow_off[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = 8 * it + (lane >> 3);
    orow_off[it] = -1;
    if ((uint32_t)(wave * 32 + r) < n) {
      const long orow = out_row(jd, jd.s1 + t0 + wave * 32 + r);
      if (orow < 0)
        *bad = 1;
      else
        orow_off[it] = orow * (long)F * OSZ + c16 * 16;
    }
  }
  uint8_t* wout = smem + (size_t)wave * 32 * kOutRow;
  uint8_t* dst = (uint8_t*)jd.dst;
  const uint16_t* vrow = (const uint16_t*)(a.state + sl.vdec_off) + (size_t)(lane & 31) * r_dec + 8 * h;
  const size_t fb_stride = (size_t)32 * r_dec;        // elements per 32-feature block

  uint4 A0[KS > 0 ? KS : 1], A1[KS > 0 ? KS : 1];
  auto load_a = [&](int fb, uint4* A) {
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = *(const uint4*)(vrow + fb * fb_stride + 16 * s);
  };
  auto block = [&](int fb, const uint4* A, int u) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, A[s]),
                                                   __builtin_bit_cast(f16x8, bfr[s]), acc, 0, 0, 0);
    // D[feature][token]: lane holds token (lane & 31), features
    // fb*32 + 8*qd + 4*h + {0..3} in acc[4*qd .. 4*qd+3].
    uint8_t* orow_l = wout + (size_t)(lane & 31) * kOutRow + u * 32 * OSZ;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int f = fb * 32 + 8 * qd + 4 * h;
      const float4 m4 = *(const float4*)(mu_l + f);
      const float o0 = __builtin_fmaf(acc[4 * qd + 0], S, m4.x);
      const float o1 = __builtin_fmaf(acc[4 * qd + 1], S, m4.y);
      const float o2 = __builtin_fmaf(acc[4 * qd + 2], S, m4.z);
      const float o3 = __builtin_fmaf(acc[4 * qd + 3], S, m4.w);
      const int col = (8 * qd + 4 * h) * OSZ;
      if (OUT32)
        *(float4*)(orow_l + col) = make_float4(o0, o1, o2, o3);
      else
        *(uint2*)(orow_l + col) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
  };
  auto store_segment = [&](int fb0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (orow_off[it] >= 0) {
        const uint4 v = *(const uint4*)(wout + (size_t)(8 * it + (lane >> 3)) * kOutRow + c16 * 16);
        *(uint4*)(dst + orow_off[it] + (size_t)fb0 * 32 * OSZ) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // F/32 is even (F is a multiple of 64): feature blocks go in pairs with
  // ping-pong basis registers.
  const int nfb = F / 32;
  load_a(0, A0);
  for (int fb = 0; fb < nfb; fb += 2) {
    load_a(fb + 1, A1);
    block(fb, A0, OUT32 ? 0 : 0);
    if (OUT32) store_segment(fb);
    if (fb + 2 < nfb) load_a(fb + 2, A0);
    block(fb + 1, A1, OUT32 ? 0 : 1);
    store_segment(OUT32 ? fb + 1 : fb);
  }
}

// Fused decode: header check, passthrough tiles and compressed tiles.
template <int KS, bool OUT32>
__global__ __launch_bounds__(kThreads) void decode_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int flag;
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const int j = find_job(a, tile);
  const JobDesc& jd = a.jobs[j];
  const DevSlot& sl = ((const DevSlot*)a.state)[jd.slot];
  const uint32_t lt = tile - jd.tile_begin;
  if (threadIdx.x == 0) flag = check_header(a, jd, sl);
  __syncthreads();
  const int st = flag;
  if (lt == 0 && threadIdx.x == 0) set_status(a, jd.status_idx, st);
  if (st != KVTC_OK) return;
  __syncthreads();
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  int bad = 0;
  if (lt >= jd.n_ctiles) {
    bad = !decode_passthrough(a, jd, lt - jd.n_ctiles);
  } else {
    const uint32_t t0 = lt * kDecTile;
    const uint32_t n = min((uint32_t)kDecTile, jd.tc - t0);
    restore_tile<KS, OUT32, false>(a, jd, sl, smem, t0, n, &bad);
  }
  if (bad) atomicExch(&flag, 1);
  __syncthreads();
  if (threadIdx.x == 0 && flag) set_status(a, jd.status_idx, KVTC_E_INVALID);
}

// Stage 1: header check, passthrough rows, records -> staging codes/scales.
template <int G>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int flag;
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const int j = find_job(a, tile);
  const JobDesc& jd = a.jobs[j];
  const DevSlot& sl = ((const DevSlot*)a.state)[jd.slot];
  const uint32_t lt = tile - jd.tile_begin;
  if (threadIdx.x == 0) flag = check_header(a, jd, sl);
  __syncthreads();
  const int st = flag;
  if (lt == 0 && threadIdx.x == 0) set_status(a, jd.status_idx, st);
  if (st != KVTC_OK) return;
  __syncthreads();
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  int bad = 0;
  if (lt >= jd.n_ctiles) {
    bad = !decode_passthrough(a, jd, lt - jd.n_ctiles);
  } else if (sl.r_eff > 0) {
    const uint32_t t0 = lt * kUnpackTile;
    const uint32_t n = min((uint32_t)kUnpackTile, jd.tc - t0);
    const int esz = a.dtype == KVTC_F32 ? 4 : 2;
    const int rb = sl.record_bytes;
    const uint8_t* recs = (const uint8_t*)jd.src + record_base(jd, a.F, esz) + (size_t)t0 * rb;
    stage_to_lds(smem, recs, (size_t)n * rb);
    __syncthreads();
    uint8_t* st8 = (uint8_t*)jd.staging;
    float2* ssg = (float2*)(st8 + align_up((size_t)jd.tc * sl.r_eff, kAlign));
    // One thread per (token, 8-component chunk).
    const int chunks = sl.r_eff / 8;
    for (int idx = threadIdx.x; idx < (int)n * chunks; idx += kThreads) {
      const int tl = idx / chunks, c = (idx % chunks) * 8;
      const uint8_t* rec = smem + (size_t)tl * rb;
      const int ag = c / G, o = c % G;
      *(uint64_t*)(st8 + (size_t)(t0 + tl) * sl.r_eff + c) = get_codes8(rec, sl, ag, o);
      if (o == 0) {
        const uint64_t raw = lds_u64(rec + 8 * ag);
        ssg[(size_t)(t0 + tl) * sl.n_act + ag] =
            make_float2(__uint_as_float((uint32_t)raw), __uint_as_float((uint32_t)(raw >> 32)));
      }
    }
  }
  if (bad) atomicExch(&flag, 1);
  __syncthreads();
  if (threadIdx.x == 0 && flag) set_status(a, jd.status_idx, KVTC_E_INVALID);
}

// Stage 2: staging -> compressed output rows.
template <int KS, bool OUT32>
__global__ __launch_bounds__(kThreads) void restore_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int flag;
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const int j = find_job(a, tile);
  const JobDesc& jd = a.jobs[j];
  const DevSlot& sl = ((const DevSlot*)a.state)[jd.slot];
  const uint32_t lt = tile - jd.tile_begin;
  if (prior_rank(a, jd.status_idx) != 0 || lt >= jd.n_ctiles) return;  // stage 1 rejected it
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  int bad = 0;
  const uint32_t t0 = lt * kDecTile;
  const uint32_t n = min((uint32_t)kDecTile, jd.tc - t0);
  restore_tile<KS, OUT32, true>(a, jd, sl, smem, t0, n, &bad);
  if (bad) atomicExch(&flag, 1);
  __syncthreads();
  if (threadIdx.x == 0 && flag) set_status(a, jd.status_idx, KVTC_E_INVALID);
}

// Test hook: stream from given codes and (shift, scale) pairs, through the
// encoder's record packing (put_group) and header/passthrough writers.
template <int G>
__global__ __launch_bounds__(kThreads) void pack_kernel(const LaunchArgs a, const uint8_t* codes,
                                                        const float2* ss) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const JobDesc& jd = a.jobs[0];
  const DevSlot& sl = ((const DevSlot*)a.state)[jd.slot];
  const uint32_t lt = tile - jd.tile_begin;
  const int esz = a.dtype == KVTC_F32 ? 4 : 2;
  const size_t row_bytes = (size_t)a.F * esz;
  if (lt == 0 && threadIdx.x == 0) {
    write_header(a, jd, sl);
    set_status(a, jd.status_idx, KVTC_OK);
  }
  if (lt >= jd.n_ctiles) {
    encode_passthrough(jd, lt - jd.n_ctiles, row_bytes);
    return;
  }
  if (sl.r_eff == 0) return;
  const uint32_t t0 = lt * kEncTile;
  const uint32_t n = min((uint32_t)kEncTile, jd.tc - t0);
  const int rb = sl.record_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);
  if ((uint32_t)tl < n) {
    const uint32_t t = t0 + tl;
    for (int ag = 0; ag < sl.n_act; ++ag) {
      uint32_t cv[G / 2];
      for (int i = 0; i < G / 2; ++i) cv[i] = codes[(size_t)t * sl.r_eff + ag * G + h * (G / 2) + i];
      const float2 p = ss[(size_t)t * sl.n_act + ag];
      put_group<G>(smem + (size_t)tl * rb, sl, ag, h, cv, p.x, p.y);
    }
  }
  __syncthreads();
  lds_to_global((uint8_t*)jd.dst + record_base(jd, a.F, esz) + (size_t)t0 * rb, smem, (size_t)n * rb);
}

// ------------------------------------------------------------- launchers ---

static dim3 grid_for(uint32_t tiles) { return dim3((tiles + 7u) / 8u * 8u); }

// Dynamic LDS above the 64 KiB default needs an explicit opt-in (gfx950 has
// 160 KiB per CU).
template <class K>
static void allow_lds(K kernel, size_t lds) {
  if (lds > 65536) hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int G, bool F32IN>
static int launch_encode_g(const LaunchArgs& a, int nb, size_t lds, hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
#define KVTC_ENC(NBV)                                                                  \
  case NBV:                                                                            \
    allow_lds(encode_kernel<NBV, G, F32IN>, lds);                                      \
    hipLaunchKernelGGL((encode_kernel<NBV, G, F32IN>), g, dim3(kThreads), lds, s, a);  \
    break;
  switch (nb) {
    KVTC_ENC(1) KVTC_ENC(2) KVTC_ENC(3) KVTC_ENC(4) KVTC_ENC(5) KVTC_ENC(6) KVTC_ENC(7) KVTC_ENC(8)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_ENC
  return (int)hipGetLastError();
}

int launch_encode(const LaunchArgs& a, int nb, int G, size_t lds, hipStream_t s) {
  const bool f32 = a.dtype == KVTC_F32;
  if (G == 16) return f32 ? launch_encode_g<16, true>(a, nb, lds, s) : launch_encode_g<16, false>(a, nb, lds, s);
  if (G == 32) return f32 ? launch_encode_g<32, true>(a, nb, lds, s) : launch_encode_g<32, false>(a, nb, lds, s);
  return (int)hipErrorInvalidValue;
}

size_t decode_lds_bytes(int r_dec, int F) { return dec_lds_bytes(r_dec, F); }

// Decode launches take the exact K-step count ks = r_dec / 16 of every job
// in the batch (the host groups jobs by it).
template <bool OUT32>
static int launch_decode_o(const LaunchArgs& a, int ks, size_t lds, bool staged, hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
#define KVTC_DEC(KV)                                                                 \
  case KV:                                                                           \
    if (staged) {                                                                    \
      allow_lds(restore_kernel<KV, OUT32>, lds);                                     \
      hipLaunchKernelGGL((restore_kernel<KV, OUT32>), g, dim3(kThreads), lds, s, a); \
    } else {                                                                         \
      allow_lds(decode_kernel<KV, OUT32>, lds);                                      \
      hipLaunchKernelGGL((decode_kernel<KV, OUT32>), g, dim3(kThreads), lds, s, a);  \
    }                                                                                \
    break;
  switch (ks) {
    KVTC_DEC(0) KVTC_DEC(1) KVTC_DEC(2) KVTC_DEC(3) KVTC_DEC(4) KVTC_DEC(5) KVTC_DEC(6)
    KVTC_DEC(7) KVTC_DEC(8) KVTC_DEC(9) KVTC_DEC(10) KVTC_DEC(11) KVTC_DEC(12) KVTC_DEC(13)
    KVTC_DEC(14) KVTC_DEC(15) KVTC_DEC(16)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_DEC
  return (int)hipGetLastError();
}

int launch_decode(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  return a.out_dtype == KVTC_F32 ? launch_decode_o<true>(a, ks, lds, false, s)
                                 : launch_decode_o<false>(a, ks, lds, false, s);
}

int launch_restore(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  return a.out_dtype == KVTC_F32 ? launch_decode_o<true>(a, ks, lds, true, s)
                                 : launch_decode_o<false>(a, ks, lds, true, s);
}

int launch_unpack(const LaunchArgs& a, int G, size_t lds, hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
  if (G == 16) {
    allow_lds(unpack_kernel<16>, lds);
    hipLaunchKernelGGL((unpack_kernel<16>), g, dim3(kThreads), lds, s, a);
  } else if (G == 32) {
    allow_lds(unpack_kernel<32>, lds);
    hipLaunchKernelGGL((unpack_kernel<32>), g, dim3(kThreads), lds, s, a);
  }
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_pack(const LaunchArgs& a, int G, size_t lds, const void* codes, const void* ss,
                hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
  if (G == 16)
    hipLaunchKernelGGL((pack_kernel<16>), g, dim3(kThreads), lds, s, a, (const uint8_t*)codes,
                       (const float2*)ss);
  else if (G == 32)
    hipLaunchKernelGGL((pack_kernel<32>), g, dim3(kThreads), lds, s, a, (const uint8_t*)codes,
                       (const float2*)ss);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace kvtc
