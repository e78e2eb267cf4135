// HIP kernels of KV-cache transform coding for gfx950 (MI355X).
//
// Method: "KV Cache Transform Coding for Compact Storage in LLM Inference"
// (gist.science, 2511.01815), section 2B (compression: subtract the mean,
// multiply by V, quantize with the DP widths, pack) and section 2C
// (decompression: dequantize, multiply by V^T, add the mean, layer by layer).
//
// Every launch covers a batch of jobs (tensors) of one shape parameter, with
// the job descriptors passed by value. Persistent grids take equal contiguous
// ranges of work units, and the blockIdx -> range map sends consecutive
// ranges to the same XCD, so one tensor's basis stays in one XCD's L2.
//
// Encode (256 threads, persistent, at most two workgroups per CU): each wave
// owns 32 tokens of a tile. The projection runs on v_mfma_f32_32x32x16_bf16
// in transposed form, D[component][token] = sum_f V'^T[component][f] *
// x[token][f], with the accumulators started at -mu V' for bf16 input (the
// mean folded into the product) and f32 input centred and split into two
// bf16 operands. Token rows go through a per-wave LDS tile (row-contiguous
// loads), basis K-slices through two shared LDS buffers, both two slices
// ahead. In the accumulator layout a lane owns one token and half of every
// group's components, so the per-(token, group) min/max needs one cross-lane
// exchange (lane ^ 32) and quantization is lane-local; codes are OR-ed into
// LDS record rows and leave in 16-byte stores.
//
// Decode, stage 1 (256 threads): one wave per block of 32 compressed tokens
// loads the block's records, stages them in LDS and builds each token's
// dequantized coefficients c_hat = shift + q * fp32(scale / k) for the 8
// components per K step it feeds to the MFMA, divided by a per-token power of
// two into fp16 (the fp16 operand keeps 11 significant bits; the scale makes
// the range irrelevant), into a staging buffer. Stage 2 (512 threads,
// persistent): D[feature][token] = sum_j V'[feature][j] * c_hat[token][j] on
// v_mfma_f32_32x32x16_f16 per 128-feature slab (V' in LDS), written as
// S_t * D + mu through LDS rows in 128-byte streaming stores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "kvtc_internal.h"

namespace kvtc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
static_assert(kWaves == kPrepWaves, "stage-1 workgroups run kThreads threads");

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
// The aligned address is formed as p minus its misalignment (not through an
// integer round trip) so the compiler still sees an LDS pointer and emits
// ds_read rather than a flat load, which would also wait for pending stores.
__device__ __forceinline__ uint64_t lds_u64(const uint8_t* p) {
  const uint32_t sh = (uint32_t)(uintptr_t)p & 3u;
  const uint32_t* b = (const uint32_t*)(p - sh);
  const uint32_t w0 = b[0], w1 = b[1], w2 = b[2];
  const uint32_t lo = __builtin_amdgcn_alignbyte(w1, w0, sh);
  const uint32_t hi = __builtin_amdgcn_alignbyte(w2, w1, sh);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Device-state slots are read through the constant address space: the
// state is never written by a kernel, so uniform reads become scalar loads.
// Vector loads of it would be counted with the token and record traffic, and
// their waits would drain every load in flight. Sub-dword fields are read
// as whole dwords (scalar loads are dword-granular).
typedef const __attribute__((address_space(4))) DevSlot CSlot;
typedef const __attribute__((address_space(4))) uint32_t CU32;
__device__ __forceinline__ CSlot& slot_of(const LaunchArgs& a, int s) { return ((CSlot*)a.state)[s]; }
__device__ __forceinline__ int slot_width(CSlot& sl, int g) {
  return (int)((((CU32*)sl.width)[g >> 2] >> (8 * (g & 3))) & 0xFFu);
}
__device__ __forceinline__ int slot_chunk(CSlot& sl, int g) {
  return (int)((((CU32*)sl.chunk_off)[g >> 1] >> (16 * (g & 1))) & 0xFFFFu);
}
static_assert(offsetof(DevSlot, width) % 4 == 0 && offsetof(DevSlot, chunk_off) % 4 == 0,
              "packed slot arrays are read as dwords");
static_assert(kMaxActGroups % 4 == 0, "packed slot arrays are read as dwords");

__device__ __forceinline__ size_t record_base(const JobDesc& jd, int F, int esz) {
  return (size_t)kHeaderBytes + (size_t)(jd.s1 + jd.w1) * F * esz;
}

__device__ void write_header(const LaunchArgs& a, const JobDesc& jd, CSlot& sl) {
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
// (Read through the constant address space: uniform scalar loads; the
// stream is not written while it is decoded.)
__device__ int check_header(const LaunchArgs& a, const JobDesc& jd, CSlot& sl) {
  CU32* h = (CU32*)jd.src;
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
// (rows [0, s') then [T - w', T)) from the KV tensor into the stream, with
// four 16-byte loads in flight per thread.
__device__ void encode_passthrough(const JobDesc& jd, uint32_t p, size_t row_bytes) {
  const uint32_t n_rows = jd.s1 + jd.w1;
  const uint32_t r0 = p * kPassRows;
  const uint32_t r1 = min(n_rows, r0 + kPassRows);
  const uint32_t vpr = (uint32_t)(row_bytes / 16);
  const uint32_t total = (r1 - r0) * vpr;
  uint8_t* dst = (uint8_t*)jd.dst + kHeaderBytes + (size_t)r0 * row_bytes;
  for (uint32_t i0 = threadIdx.x; i0 < total; i0 += 4 * kThreads) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + u * kThreads;
      if (i < total) {
        const uint32_t r = r0 + i / vpr;
        const uint32_t src_row = r < jd.s1 ? r : jd.T - jd.w1 + (r - jd.s1);
        v[u] = ((const u32x4*)((const uint8_t*)jd.src + (size_t)src_row * row_bytes))[i % vpr];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + u * kThreads;
      if (i < total) ((u32x4*)dst)[i] = v[u];
    }
  }
}

// Decode: copy passthrough rows [p*PR, ...) of the stream's row list to the
// output, converting the element type if needed; every thread of the
// workgroup (NT threads) calls it (rows_lds: PR longs of LDS). The output row of
// each stream row is looked up once; the copy keeps four 16-byte loads in
// flight per thread. Returns false if a block table entry was bad.
template <int NT, int PR = kPassRows>
__device__ bool decode_passthrough(const LaunchArgs& a, const JobDesc& jd, uint32_t p, long* rows_lds) {
  const int F = a.F;
  const uint32_t n_rows = jd.s1 + jd.w1;
  const uint32_t r0 = p * PR;
  const uint32_t nr = min(n_rows, r0 + PR) - r0;
  const int in_esz = a.dtype == KVTC_F32 ? 4 : 2;
  const int out_esz = a.out_dtype == KVTC_F32 ? 4 : 2;
  const uint8_t* src = (const uint8_t*)jd.src + kHeaderBytes + (size_t)r0 * F * in_esz;
  if (threadIdx.x < nr) {
    const uint32_t r = r0 + threadIdx.x;
    rows_lds[threadIdx.x] = out_row(jd, r < jd.s1 ? r : jd.T - jd.w1 + (r - jd.s1));
  }
  __syncthreads();
  bool ok = true;
  if (a.dtype == a.out_dtype) {
    const uint32_t vpr = (uint32_t)F * in_esz / 16;          // 16-byte vectors per row
    const uint32_t total = nr * vpr;
    for (uint32_t i0 = threadIdx.x; i0 < total; i0 += 4 * NT) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = i0 + u * NT;
        if (i < total) v[u] = ((const u32x4*)src)[i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = i0 + u * NT;
        if (i < total) {
          const uint32_t rr = i / vpr;
          const long orow = rows_lds[rr];
          if (orow < 0) {
            ok = false;
          } else {
            ((u32x4*)((uint8_t*)jd.dst + (size_t)orow * F * out_esz))[i - rr * vpr] = v[u];
          }
        }
      }
    }
  } else {
    const uint32_t total = nr * (uint32_t)F;
    for (uint32_t i = threadIdx.x; i < total; i += NT) {
      const uint32_t rr = i / (uint32_t)F;
      const int c = (int)(i - rr * (uint32_t)F);
      const long orow = rows_lds[rr];
      if (orow < 0) { ok = false; continue; }
      if (a.dtype == KVTC_BF16) {  // bf16 -> f32, exact
        const uint16_t b = ((const uint16_t*)src)[i];
        ((float*)jd.dst)[(size_t)orow * F + c] = bf16_to_f32(b);
      } else {                     // f32 -> bf16, nearest even
        const float f = ((const float*)src)[i];
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
__device__ __forceinline__ void put_group(uint8_t* rec, CSlot& sl, int a, int h,
                                          const uint32_t* codes, float shift, float scale) {
  const int w = slot_width(sl, a);
  const int half_bytes = (G / 2) * w / 8;
  uint8_t* p = rec + slot_chunk(sl, a) + h * half_bytes;
  if (G == 16) {
    lds_store_bytes(p, pack_codes(codes, 8, w), w);
  } else {
    lds_store_bytes(p, pack_codes(codes, 8, w), w);
    lds_store_bytes(p + w, pack_codes(codes + 8, 8, w), w);
  }
  if (h == 0) {  // rec is 4-byte aligned (padded_stride)
    ((uint32_t*)(rec + 8 * a))[0] = __float_as_uint(shift);
    ((uint32_t*)(rec + 8 * a))[1] = __float_as_uint(scale);
  }
}

// Copy n records of rb bytes from LDS rows of stride rbp into the contiguous
// stream at dst (16-byte aligned): 16-byte stores gathered from 4-byte (rb %
// 4 == 0) or 2-byte pieces, then a byte tail.
__device__ void records_to_global(uint8_t* dst, const uint8_t* lds, uint32_t n, int rb, int rbp) {
  const uint32_t total = n * (uint32_t)rb;
  const uint32_t nv = total / 16;
  const float inv = 1.0f / (float)rb;
  auto locate = [&](uint32_t j, uint32_t& row, uint32_t& col) {
    row = (uint32_t)((float)j * inv);
    while (row * (uint32_t)rb > j) --row;
    while ((row + 1) * (uint32_t)rb <= j) ++row;
    col = j - row * (uint32_t)rb;
  };
  for (uint32_t v = threadIdx.x; v < nv; v += kThreads) {
    uint32_t row, col;
    locate(v * 16, row, col);
    uint32_t w[4];
    if ((rb & 3) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = *(const uint32_t*)(lds + row * rbp + col);
        col += 4;
        if (col >= (uint32_t)rb) { col = 0; ++row; }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = *(const uint16_t*)(lds + row * rbp + col);
        col += 2;
        if (col >= (uint32_t)rb) { col = 0; ++row; }
        uint32_t hi = *(const uint16_t*)(lds + row * rbp + col);
        col += 2;
        if (col >= (uint32_t)rb) { col = 0; ++row; }
        w[i] = lo | (hi << 16);
      }
    }
    *(uint4*)(dst + (size_t)v * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (uint32_t j = nv * 16 + threadIdx.x; j < total; j += kThreads) {
    uint32_t row, col;
    locate(j, row, col);
    dst[j] = lds[row * rbp + col];
  }
}

// The 8 codes of components [o, o + 8) of active group a from a record:
// one byte per code in a 64-bit word.
__device__ __forceinline__ uint64_t get_codes8(const uint8_t* rec, CSlot& sl, int a, int o) {
  const int w = slot_width(sl, a);
  const uint64_t bits = lds_u64(rec + slot_chunk(sl, a) + (o * w) / 8);
  const uint64_t mask = (1ull << w) - 1ull;
  uint64_t out = 0;
  for (int j = 0; j < 8; ++j) out |= ((bits >> (j * w)) & mask) << (8 * j);
  return out;
}

// Make this wave's LDS writes visible to its own lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// --------------------------------------------------------------- encode ---

// Compressed rows carry their own index space of kEncBlk-token blocks
// (JobDesc::cblk_begin): the blocks of every job with records, job after job.
__device__ __forceinline__ int find_cblk_job(const LaunchArgs& a, uint32_t b) {
  int j = 0;
  for (int i = 1; i < a.n_jobs; ++i)
    if (a.jobs[i].cblk_begin <= b) j = i;
  return j;
}
// The job of block b >= the first block of job j: j moved forward (a
// workgroup's blocks are contiguous, so this is usually zero or one step).
__device__ __forceinline__ int next_cblk_job(const LaunchArgs& a, int j, uint32_t b) {
  while (j + 1 < a.n_jobs && a.jobs[j + 1].cblk_begin <= b) ++j;
  return j;
}

// The value of lane l ^ 32 (the other half-wave), through
// v_permlane32_swap: with x in both operands the first result holds the low
// half in both halves, the second the high half in both.
__device__ __forceinline__ float xor32(float x, int h) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

// Quantize the projected tile held in acc (acc[b][i]: component
// 32b + 8(i/4) + 4h + i%4 of token tl) into the token's LDS record row rec,
// which the caller has zeroed. Lane h holds, of each group, the runs of four
// components 8m + 4h .. + 3 (m < G/8): their codes occupy bits
// [(8m + 4h) w, (8m + 4h + 4) w) of the group's chunk and are merged into
// the record with at most two 32-bit ORs per run (runs of the two lanes can
// share a word).
template <int NB, int G>
__device__ __forceinline__ void quantize_tile(const f32x16 (&acc)[NB], CSlot& sl, uint8_t* rec,
                                              int h, bool tok_ok) {
  // A group of G components is the item range [(G/2) * sg, (G/2) * (sg + 1))
  // of block b with sg = a % (32/G).
  constexpr int SUB = 32 / G;
  uint32_t* const rw = (uint32_t*)rec;   // rec is 4-byte aligned (padded_stride)
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
        mn = fminf(mn, xor32(mn, h));
        mx = fmaxf(mx, xor32(mx, h));
        const int w = slot_width(sl, ag);
        const float k = (float)((1 << w) - 1);
        const float scale = mx - mn;
        const float inv = scale > 0.f ? k / scale : 0.f;
        const uint32_t base = 8u * slot_chunk(sl, ag);   // chunk bit offset in the record
#pragma unroll
        for (int m = 0; m < G / 8; ++m) {
          uint32_t run = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = v[4 * m + e] - mn;
            const float u = d * inv;
            const float r = fminf(fmaxf(__builtin_rintf(u), 0.f), k);
            run |= (uint32_t)r << (e * w);
          }
          const uint32_t pos = base + (uint32_t)(8 * m + 4 * h) * (uint32_t)w;
          const uint32_t sh = pos & 31u;
          if (tok_ok) {
            atomicOr(rw + (pos >> 5), run << sh);
            if (sh + 4u * (uint32_t)w > 32u) atomicOr(rw + (pos >> 5) + 1, run >> (32u - sh));
          }
        }
        if (tok_ok && h == 0) {
          rw[2 * ag] = __float_as_uint(mn);
          rw[2 * ag + 1] = __float_as_uint(scale);
        }
      }
      // One group at a time: interleaving them only raises register pressure.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Persistent encode. Each workgroup first writes the headers and passthrough
// units u = g, g + grid, ... of the launch, then projects, quantizes and
// packs an equal contiguous range of the compressed 32-token blocks, as
// tiles of up to four blocks of one job. Its four waves take a block of a
// tile each; the K loop walks slices of kEncKS features.
// The slice pipeline runs across tile boundaries: a load cursor two slices
// ahead of the computation moves on into the next tile of the range, so the
// loads of a tile's first slices are in flight during the previous tile's
// quantization, and the pipeline fills once per workgroup.
template <int NB, int G, bool F32IN, bool ODD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(!F32IN && NB <= 3 ? 3 : 1))) void encode_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t g = logical_tile();
  const int F = a.F;
  constexpr int esz = F32IN ? 4 : 2;
  const size_t row_bytes = (size_t)F * esz;
  for (uint32_t u = g; u < a.total_tiles; u += gridDim.x) {
    const JobDesc& jd = a.jobs[find_job(a, u)];
    const uint32_t lt = u - jd.tile_begin;
    if (lt == 0 && threadIdx.x == 0) {
      write_header(a, jd, slot_of(a, jd.slot));
      set_status(a, jd.status_idx, KVTC_OK);
    }
    if (lt >= jd.n_ctiles) encode_passthrough(jd, lt - jd.n_ctiles, row_bytes);
  }
  // This workgroup's blocks [b_begin, b_end), taken as tiles of up to
  // kEncWaves blocks of one job (tile_end); equal block counts per
  // workgroup keep them busy until the end of the launch.
  const uint32_t B = a.total_cblks;
  const uint32_t b_begin = (uint32_t)((uint64_t)B * g / gridDim.x);
  const uint32_t b_end = (uint32_t)((uint64_t)B * (g + 1) / gridDim.x);
  if (b_begin >= b_end) return;
  auto tile_end = [&](int j, uint32_t b) -> uint32_t {
    const JobDesc& jd = a.jobs[j];
    const uint32_t job_end = jd.cblk_begin + (jd.tc + kEncBlk - 1) / kEncBlk;
    return min(min(b + (uint32_t)kEncWaves, job_end), b_end);
  };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);            // token within the tile
  static_assert(kEncWaves * 64 == kThreads, "one wave per 32 tokens of a tile");

  // LDS: two basis K-slices [32 * NB][kEncRowPad] bf16, the wave's token
  // tiles [32][kEncRowPad] bf16 (one; for f32 input two, high and low part),
  // then for f32 input the mean (F fp32). Basis slices and token rows are
  // loaded from memory two slices ahead of their use: during slice i the
  // loads of slice i + 2 are issued, and at the end of slice i the token rows
  // of slice i + 1 go to the wave's token tiles and basis slice i + 1 to the
  // other basis buffer (last read in slice i - 1, before the barrier that
  // ended it). After a tile's last slice the records are assembled in LDS
  // from offset 0, then slice 0 of the next tile is staged. Loads past the
  // range's last slice re-read it, so every slice issues the same loads and
  // the waits count exactly.
  //
  // The projection c = (x - mu) V' is taken as x V' - mu V': a bf16 token is
  // an exact MFMA operand, so only the fp32 sums round, and mu V' (fp64,
  // rounded once, in the device state) is subtracted per component at the
  // end. An f32 token is centred in fp32 and split into two bf16 operands
  // hi = bf16(x - mu), lo = bf16(x - mu - hi), both multiplied.
  constexpr int slice_elems = 32 * NB * kEncRowPad;
  constexpr int XT = 32 * kEncRowPad;   // elements per token tile
  uint16_t* const vbase = (uint16_t*)smem;
  uint16_t* const xs = (uint16_t*)(smem + 2 * enc_basis_bytes(NB) + wave * enc_xtile_bytes(F32IN));
  float* const mu_l = (float*)(smem + 2 * enc_basis_bytes(NB) + kEncWaves * enc_xtile_bytes(F32IN));
  const int n_sl = F / kEncKS;   // odd exactly when ODD (the host picks the kernel)

  // Load cursor: tile lc, slice lk; the tile's basis and token row offsets.
  // Rows past the tile's last token re-read its first row; their results
  // are dropped.
  constexpr int CH = kEncKS * esz / 16;   // 16-byte chunks per row segment
  constexpr int RPI = 64 / CH;            // rows per load instruction
  constexpr int NI = 32 / RPI;            // load instructions per slice
  constexpr int EPC = 16 / esz;           // features per chunk
  const int cx = lane % CH;
  uint32_t lbe;       // end block of the load cursor's tile
  int lk = 0;
  const int j_begin = find_cblk_job(a, b_begin);
  int lj = j_begin;   // the load cursor's job
  const uint16_t* l_venc;
  const uint8_t* l_x;
  const float* l_mu;
  uint32_t xoff[NI];
  auto cursor_tile = [&](uint32_t b) __attribute__((always_inline)) {
    lj = next_cblk_job(a, lj, b);
    const JobDesc& jd = a.jobs[lj];
    CSlot& sl = slot_of(a, jd.slot);
    lbe = tile_end(lj, b);
    const uint32_t t0 = (b - jd.cblk_begin) * kEncBlk;
    const uint32_t n = min((lbe - b) * kEncBlk, jd.tc - t0);
    l_venc = (const uint16_t*)(a.state + sl.venc_off);
    l_mu = (const float*)(a.state + sl.mu_off);
    l_x = (const uint8_t*)jd.src + (size_t)(jd.s1 + t0) * row_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t r = (uint32_t)(wave * 32 + i * RPI + lane / CH);
      xoff[i] = (r < n ? r : 0u) * (uint32_t)row_bytes + (uint32_t)cx * 16u;
    }
  };
  auto cursor_next = [&]() __attribute__((always_inline)) {
    if (lk + 1 < n_sl) {
      ++lk;
    } else if (lbe < b_end) {
      lk = 0;
      cursor_tile(lbe);
    }
  };
  cursor_tile(b_begin);

  // Slice copy: a slice holds 32 * NB rows of kEncKS features, 32 * NB * 8
  // vectors of 16 bytes, so thread t moves vectors t + q * kThreads, q < NB,
  // with no predicate. Every job of a launch has r_enc = 32 * NB; rows >=
  // r_eff are zero in the device state.
  typedef uint32_t vregs_t __attribute__((ext_vector_type(4 * NB)));
#define KVTC_LOAD_SLICE(V)                                                              \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                      \
    const int idx = (int)threadIdx.x + q * kThreads;                                    \
    const uint4 v = *(const uint4*)(l_venc + (size_t)(idx / (kEncKS / 8)) * F +          \
                                    lk * kEncKS + (idx % (kEncKS / 8)) * 8);            \
    V[4 * q] = v.x;                                                                     \
    V[4 * q + 1] = v.y;                                                                 \
    V[4 * q + 2] = v.z;                                                                 \
    V[4 * q + 3] = v.w;                                                                 \
  }
#define KVTC_STORE_SLICE(V, BUF)                                                     \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                   \
    const int idx = (int)threadIdx.x + q * kThreads;                                 \
    *(uint4*)((BUF) + (idx / (kEncKS / 8)) * kEncRowPad + (idx % (kEncKS / 8)) * 8) = \
        make_uint4(V[4 * q], V[4 * q + 1], V[4 * q + 2], V[4 * q + 3]);              \
  }
#define KVTC_LOAD_X(DST) \
  _Pragma("unroll") for (int i = 0; i < NI; ++i) DST[i] = *(const u32x4*)(l_x + xoff[i] + (size_t)lk * kEncKS * esz);
  // Rows of one slice into the wave's token tiles: row i * RPI + lane / CH,
  // features cx * EPC .. + EPC. bf16 rows are stored as loaded; f32 rows are
  // centred with the mean of their tile's job (mu_l, staged with slice 0).
  auto stage_x = [&](int k0, const u32x4 (&xr)[NI]) __attribute__((always_inline)) {
    if (!F32IN) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *(u32x4*)(xs + (i * RPI + lane / CH) * kEncRowPad + cx * EPC) = xr[i];
    } else {
      const float4 m = *(const float4*)(mu_l + k0 + cx * EPC);
      const float mv[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint32_t hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float d0 = __uint_as_float(xr[i][2 * e]) - mv[2 * e];
          const float d1 = __uint_as_float(xr[i][2 * e + 1]) - mv[2 * e + 1];
          hi[e] = pack_bf16x2(d0, d1);
          lo[e] = pack_bf16x2(d0 - bf16_to_f32(hi[e] & 0xFFFFu), d1 - bf16_to_f32(hi[e] >> 16));
        }
        uint16_t* dst = xs + (i * RPI + lane / CH) * kEncRowPad + cx * EPC;
        *(uint2*)dst = make_uint2(hi[0], hi[1]);
        *(uint2*)(dst + XT) = make_uint2(lo[0], lo[1]);
      }
    }
  };
  // Slice 0 of a tile: its job's mean (f32 input), basis and token rows.
  auto stage_first = [&](const float* mu, const u32x4 (&xr)[NI], const vregs_t& v)
      __attribute__((always_inline)) {
    if (F32IN) {
      for (int i = threadIdx.x; i < F / 4; i += kThreads) ((float4*)mu_l)[i] = ((const float4*)mu)[i];
      __syncthreads();
    }
    stage_x(0, xr);
    KVTC_STORE_SLICE(v, vbase)
    __syncthreads();
  };

  // acc[b][i] holds component 32b + 8(i/4) + 4h + i%4 of token tl. It
  // starts at -mu V' for bf16 input (the x V' - mu V' form), at 0 for f32.
  f32x16 acc[NB];
  auto init_acc = [&](int j) __attribute__((always_inline)) {
    if (F32IN) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
    } else {
      // Scalar loads (constant address space): items 32b + 8q + e of the
      // low half-wave, + 4 for the high one.
      CSlot& sl = slot_of(a, a.jobs[j].slot);
      CU32* cmu = (CU32*)(a.state + sl.cmu_off);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(cmu[32 * b + 8 * q + e]);
            const float hi = __uint_as_float(cmu[32 * b + 8 * q + 4 + e]);
            acc[b][4 * q + e] = -(h ? hi : lo);
          }
    }
  };
  // One slice: run the K steps of slice it (token tile, basis buffer it % 2;
  // K step s takes features 16s + 8h .. +8 of the slice), issue the loads at
  // the load cursor (basis into vl, tokens into xl, both free since the end
  // of slice it - 1; mul is the mean of the tile they belong to), then,
  // unless it is the tile's last slice,
  // stage slice it + 1 (tokens xn, basis vs). The caller alternates the
  // register sets, so no register is copied and every wait is for loads
  // issued one slice earlier.
  auto step = [&](int it, const u32x4 (&xn)[NI], u32x4 (&xl)[NI], vregs_t& vl, vregs_t& vs,
                  const float*& mul) __attribute__((always_inline)) {
    const uint16_t* vsl = vbase + (it & 1) * slice_elems;
#pragma unroll
    for (int s = 0; s < kEncKS / 16; ++s) {
      const int xo = (lane & 31) * kEncRowPad + 16 * s + 8 * h;
      const bf16x8 bx = __builtin_bit_cast(bf16x8, *(const uint4*)(xs + xo));
      bf16x8 bl;
      if (F32IN) bl = __builtin_bit_cast(bf16x8, *(const uint4*)(xs + XT + xo));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *(const uint4*)(vsl + (b * 32 + (lane & 31)) * kEncRowPad + 16 * s + 8 * h));
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bx, acc[b], 0, 0, 0);
        if (F32IN) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc[b], 0, 0, 0);
      }
    }
    // The loads go after the MFMA issue: when the memory pipeline is backed
    // up, issuing them stalls the wave, and the MFMAs then run meanwhile.
    __builtin_amdgcn_sched_barrier(0);
    KVTC_LOAD_SLICE(vl)
    KVTC_LOAD_X(xl)
    mul = l_mu;
    cursor_next();
    // The token tile is private to the wave: its reads above come before the
    // writes below in the wave's LDS order. After a tile's last slice this
    // stages the next tile's slice 0, which the records then overwrite; it
    // is staged again from the same registers after them.
    wave_lds_sync();
    stage_x(((it + 1) % n_sl) * kEncKS, xn);
    KVTC_STORE_SLICE(vs, vbase + ((it + 1) & 1) * slice_elems)
    __syncthreads();
  };

  u32x4 x0[NI], x1[NI];
  vregs_t v0, v1;
  const float *mu0 = l_mu, *mu1;   // the mean of the tile in x0 / x1
  KVTC_LOAD_SLICE(v0)
  KVTC_LOAD_X(x0)
  cursor_next();
  mu1 = l_mu;
  KVTC_LOAD_SLICE(v1)
  KVTC_LOAD_X(x1)
  cursor_next();
  init_acc(j_begin);
  stage_first(mu0, x0, v0);
  int cj = j_begin;   // the computed tile's job
  for (uint32_t b = b_begin, te; b < b_end; b = te) {
    cj = next_cblk_job(a, cj, b);
    te = tile_end(cj, b);
    const JobDesc& jd = a.jobs[cj];
    CSlot& sl = slot_of(a, jd.slot);
    const uint32_t t0 = (b - jd.cblk_begin) * kEncBlk;
    const uint32_t n = min((te - b) * kEncBlk, jd.tc - t0);
    // The loop runs whole pairs of steps and an odd last slice follows it,
    // so the loop is only re-entered after a pair; with the parity fixed at
    // compile time every path into the loop has the same loads in flight and
    // the waits the compiler derives at its head cover just those.
    int it = 0;
    for (; it + 1 < n_sl; it += 2) {
      step(it, x1, x0, v0, v1, mu0);
      step(it + 1, x0, x1, v1, v0, mu1);
    }
    if (ODD) step(it, x1, x0, v0, v1, mu0);
    __syncthreads();  // every wave is done with the slices in LDS
    const int rb = sl.record_bytes;
    const int rbp = padded_stride(rb);
    {
      // Zero the wave's 32 record rows (16-byte aligned: rbp % 4 == 0).
      u32x4* z = (u32x4*)(smem + (size_t)wave * 32 * rbp);
      const int nz = 32 * rbp / 16;
      for (int i = lane; i < nz; i += 64) z[i] = (u32x4){0u, 0u, 0u, 0u};
      wave_lds_sync();
    }
    quantize_tile<NB, G>(acc, sl, smem + (size_t)tl * rbp, h, (uint32_t)tl < n);
    if (te < b_end) init_acc(next_cblk_job(a, cj, te));
    __syncthreads();
    records_to_global((uint8_t*)jd.dst + record_base(jd, F, esz) + (size_t)t0 * rb, smem, n, rb, rbp);
    if (te < b_end) {
      __syncthreads();  // the records are out of LDS
      if (ODD) {
        // Odd slice count: the next tile's slice 0 is in (x1, v1), slice 1
        // in (x0, v0); swap so the tile starts like the first one.
        stage_first(mu1, x1, v1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const u32x4 t = x0[i];
          x0[i] = x1[i];
          x1[i] = t;
        }
        const vregs_t t = v0;
        v0 = v1;
        v1 = t;
        mu1 = mu0;
      } else {
        stage_first(mu0, x0, v0);
      }
    }
  }
#undef KVTC_LOAD_SLICE
#undef KVTC_STORE_SLICE
#undef KVTC_LOAD_X
}

// --------------------------------------------------------------- decode ---
//
// Decode runs in two kernels. Stage 1 (prep) turns each token's record into
// the MFMA B operands of the reconstruction: the dequantized coefficients
// c_hat / S_t as fp16, in MFMA lane order, with S_t a per-token power of two,
// written to a staging buffer. Stage 2 (gemm) computes x_hat = S_t * (V' B) +
// mu for every compressed row, a tall-skinny product whose cost is writing
// the output. Dequantizing once per token in stage 1 keeps that work out of
// stage 2, whose tiles each cover a slab of features.

// Per-token power-of-two scale: S = 2^(e - 14) where 2^e <= max |c_hat| over
// the token's groups < 2^(e+1), so the fp16 operand peaks in [2^14, 2^15).
__device__ __forceinline__ void token_scale(float m, float& S, float& Sinv) {
  int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
  if (m == 0.f) e = 14;
  e = max(min(e, 100), -100);
  S = __uint_as_float((uint32_t)(127 + e - 14) << 23);
  Sinv = __uint_as_float((uint32_t)(127 + 14 - e) << 23);
}

// fp32(scale / k) for k = 2^w - 1 from rk = fp32(1 / k): the product and one
// fma correction (the residual scale - q k is exact in an fma), which gives
// the correctly rounded quotient except in rare double-rounding cases, and
// exactly whenever the quotient is representable (the decode tolerance does
// not depend on the last bit; both decode routes share this function).
__device__ __forceinline__ float div_by_levels(float scale, float kf, float rk) {
  const float q = scale * rk;
  return __builtin_fmaf(__builtin_fmaf(-q, kf, scale), rk, q);
}

// B fragment of 8 components of a group of width W from packed record bits
// (code j at bits [j W, j W + W), LSB first): c_hat = shift + q * step,
// step = fp32(scale / k), times the power of two Sinv, as packed fp16.
// Sinv is folded into the fma operands; scaling by a power of two is exact,
// so the rounded results are those of the unscaled fma times Sinv. The bit
// offsets are constants, so each code is one field extract (two where it
// straddles the 32-bit halves).
template <int W>
__device__ __forceinline__ uint4 frag_w(uint64_t bits, float step, float sh) {
  constexpr uint32_t mask = (1u << W) - 1u;
  const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j * W;
    uint32_t v;
    if (p + W <= 32)
      v = (lo >> p) & mask;
    else if (p >= 32)
      v = (hi >> (p - 32)) & mask;
    else
      v = __builtin_amdgcn_alignbit(hi, lo, p) & mask;
    q[j] = (float)v;
  }
  uint32_t pk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pk[j] = pack_f16x2(__builtin_fmaf(q[2 * j], step, sh), __builtin_fmaf(q[2 * j + 1], step, sh));
  return make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// The same for a width w in 1..8 known only at run time (uniform across the
// wave: one branch per fragment); kf = 2^w - 1 and rk = fp32(1 / kf).
__device__ __forceinline__ uint4 frag_from_bits(uint64_t bits, float shift, float scale, int w,
                                                float kf, float rk, float Sinv) {
  const float step = div_by_levels(scale, kf, rk) * Sinv;
  const float sh = shift * Sinv;
  switch (w) {
    case 1: return frag_w<1>(bits, step, sh);
    case 2: return frag_w<2>(bits, step, sh);
    case 3: return frag_w<3>(bits, step, sh);
    case 4: return frag_w<4>(bits, step, sh);
    case 5: return frag_w<5>(bits, step, sh);
    case 6: return frag_w<6>(bits, step, sh);
    case 7: return frag_w<7>(bits, step, sh);
    default: return frag_w<8>(bits, step, sh);
  }
}

// Stage 1, one launch over a batch of jobs. First the header and
// passthrough units (kPrepPassRows rows each; job j owns max(1, units) of
// them from cblk_begin, and its first one records the header check in the
// job's status word), split evenly over the workgroups so they add little to
// any one; then one wave per block of kDecTok compressed tokens (block
// tile_begin + c of job j is the c-th block of its records): the wave loads
// the block's records with coalesced 16-byte loads (all in flight at once),
// stores them into its LDS rows (stride rb + 16 if rb % 16 == 0, which keeps
// a vector inside one row and spreads the rows over the banks; contiguous
// otherwise), and builds the B operands and token scales of its 32 tokens,
// stg_block_bytes(KS) bytes of staging per block. No workgroup barrier
// follows the passthrough units: the waves run on their own.
template <int KS>
__global__ __launch_bounds__(kThreads) void prep_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int flag;
  constexpr int KA = KS > 0 ? KS : 1;
  // 16-byte record vectors per lane for a block of the widest record this
  // K-step count allows (every active group of width <= 8 adds at most
  // 8 + G bytes per G / 16 K steps: rb <= 24 KS).
  constexpr int NV = (kDecTok * 24 * KA / 16 + 63) / 64;
  const uint32_t g = logical_tile(), ng = gridDim.x;
  {
    const uint32_t P = a.total_cblks;
    const uint32_t p_end = (uint32_t)((uint64_t)P * (g + 1) / ng);
    for (uint32_t p = (uint32_t)((uint64_t)P * g / ng); p < p_end; ++p) {
      int j = 0;
      for (int i = 1; i < a.n_jobs; ++i)
        if (a.jobs[i].cblk_begin <= p) j = i;
      const JobDesc& jd = a.jobs[j];
      CSlot& sl = slot_of(a, jd.slot);
      const uint32_t lp = p - jd.cblk_begin;
      const int st = check_header(a, jd, sl);   // uniform
      if (lp == 0 && threadIdx.x == 0) set_status(a, jd.status_idx, st);
      if (st != KVTC_OK) continue;
      if (threadIdx.x == 0) flag = 0;
      __syncthreads();
      bool ok = true;
      if (lp * kPrepPassRows < jd.s1 + jd.w1)
        ok = decode_passthrough<kThreads, kPrepPassRows>(a, jd, lp, (long*)smem);
      if (!ok) atomicExch(&flag, 1);
      __syncthreads();
      if (threadIdx.x == 0 && flag) set_status(a, jd.status_idx, KVTC_E_INVALID);
      __syncthreads();   // row list and flag are free for the next unit
    }
  }
  const int lane = threadIdx.x & 63, t = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t b = g * kWaves + wave;
  if (b >= a.total_tiles || KS == 0) return;
  const int j = find_job(a, b);
  const JobDesc& jd = a.jobs[j];
  CSlot& sl = slot_of(a, jd.slot);
  if (check_header(a, jd, sl) != KVTC_OK) return;   // reported by the job's first unit
  const uint32_t c = b - jd.tile_begin;
  const uint32_t nrec = min((uint32_t)kDecTok, jd.tc - c * kDecTok);
  const int rb = sl.record_bytes, rbp = dec_rec_stride(rb);
  // row of record byte q: (q * mrb) >> 24 = q / rb exactly for q < 2^24 / rb
  const uint32_t mrb = (0xFFFFFFu + (uint32_t)rb) / (uint32_t)rb;
  const uint32_t nbytes = nrec * (uint32_t)rb, nvv = nbytes / 16u;
  const uint8_t* rec = (const uint8_t*)jd.src + record_base(jd, a.F, a.dtype == KVTC_F32 ? 4 : 2) +
                       (size_t)c * kDecTok * rb;
  uint8_t* rows = smem + kPrepRowsOff + (size_t)wave * a.wave_lds;
  u32x4 x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if ((uint32_t)(64 * i) < nvv)   // uniform
      x[i] = *(const u32x4*)(rec + (size_t)min((uint32_t)(lane + 64 * i), nvv - 1u) * 16);
  // Byte q of the block's records goes to LDS byte q + (q / rb) * (rbp - rb).
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t q = (uint32_t)(lane + 64 * i) * 16u;
    if ((uint32_t)(64 * i) < nvv && q < nbytes - 15u)
      *(u32x4*)(rows + q + ((q * mrb) >> 24) * (uint32_t)(rbp - rb)) = x[i];
  }
  for (uint32_t q = nvv * 16u + lane; q < nbytes; q += 64) rows[q] = rec[q];   // ragged end (rbp == rb)
  wave_lds_sync();
  // K step s: components 16 s + 8 h .. + 8 of active group ag = 16 s / G
  // (both halves lie in one group since G >= 16, so the group, its width and
  // the reciprocal of its level count are uniform); their w-bit codes start at
  // byte off of the record, the group's (shift, scale) at byte 8 ag.
  const bool tok_ok = (uint32_t)t < nrec;
  const uint8_t* r = rows + (tok_ok ? t : 0) * rbp;
  const int G = sl.G;
  float2 ps[KA];
  float m = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint64_t q = lds_u64(r + 8 * (16 * s / G));   // rows are 2-byte aligned
    ps[s] = make_float2(__uint_as_float((uint32_t)q), __uint_as_float((uint32_t)(q >> 32)));
    // every active group has a component among the K steps, so both lanes
    // of a token see the same maximum
    m = fmaxf(m, fmaxf(fabsf(ps[s].x), fabsf(ps[s].x + ps[s].y)));
  }
  float S, Sinv;
  token_scale(m, S, Sinv);
  uint8_t* blk = (uint8_t*)jd.staging + (size_t)c * stg_block_bytes(KS);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ag = 16 * s / G;
    const int w = slot_width(sl, ag);
    const float kf = (float)((1 << w) - 1);
    const int off = slot_chunk(sl, ag) + ((16 * s + 8 * h - ag * G) * w) / 8;
    const uint4 f = tok_ok ? frag_from_bits(lds_u64(r + off), ps[s].x, ps[s].y, w, kf, 1.0f / kf, Sinv)
                           : make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)(blk + s * 1024 + lane * 16) = f;
  }
  if (h == 0) *(float*)(blk + KS * 1024 + t * 4) = tok_ok ? S : 1.f;
}

// Stage 2 segment: features [f0, f0 + FS) x blocks [c_lo, c_hi) of kDecTok
// compressed tokens of one job. The slab of V' (fp16, FS rows of r_dec,
// padded by 16 bytes per row) and mu stay in LDS; each wave then runs on its
// own over every fourth block: it loads the block's B operands and
// scales (the next block's are in flight meanwhile), runs FS / 32 x KS
// MFMAs D[feature][token], forms S_t * D + mu and stores it through its LDS
// staging rows as 128-byte segments. Every store is issued (rows past the
// tile, or with a bad block table entry, go to the workspace sink), so the
// number of memory operations per block is fixed and the wait for the next
// block's operands never covers this block's stores.
template <int KS, bool OUT32>
__device__ void gemm_segment(const LaunchArgs& a, int j, uint32_t slab, uint32_t c_lo, uint32_t c_hi,
                             uint8_t* smem) {
  constexpr int FS = gemm_features(KS);
  constexpr int NFB = FS / 32;
  constexpr int OSZ = OUT32 ? 4 : 2;
  constexpr int BPS = 128 / (32 * OSZ);           // feature blocks per 128-byte segment
  constexpr int KA = KS > 0 ? KS : 1;
  constexpr int AST = KS * 32 + 16;               // LDS bytes per V' row
  const JobDesc& jd = a.jobs[j];
  CSlot& sl = slot_of(a, jd.slot);
  if (prior_rank(a, jd.status_idx) != 0) return;  // stage 1 rejected it
  const int F = a.F;
  const int f0 = (int)slab * FS;
  const uint32_t t0 = 0;
  const int lane = threadIdx.x & 63, h = lane >> 5, c16 = lane & 7;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  uint8_t* As = smem;
  float* mu_s = (float*)(smem + FS * AST);
  uint8_t* stg = smem + FS * AST + FS * 4 + wave * kDecTok * kOutRow;
  {
    const int r_dec = sl.r_dec;
    const uint8_t* vdec = a.state + sl.vdec_off;
    for (int i = threadIdx.x; i < FS * 2 * KS; i += kGemmThreads) {
      const int row = i / (2 * KS), c = i - row * (2 * KS);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (f0 + row < F) v = *(const uint4*)(vdec + ((size_t)(f0 + row) * r_dec + 8 * c) * 2);
      *(uint4*)(As + row * AST + 16 * c) = v;
    }
    const float* mu = (const float*)(a.state + sl.mu_off);
    for (int i = threadIdx.x; i < FS; i += kGemmThreads) mu_s[i] = f0 + i < F ? mu[f0 + i] : 0.f;
  }
  __syncthreads();

  const uint8_t* stg_job = (const uint8_t*)jd.staging;
  constexpr size_t BB = stg_block_bytes(KS);
  const uint32_t tb0 = t0 / kDecTok;
  uint8_t* dst = (uint8_t*)jd.dst;
  uint8_t* sink = a.sink + c16 * 16;
  int bad = 0;
  // Job fields used per block, held in registers.
  const uint32_t tc = jd.tc, s1 = jd.s1;
  const int32_t* btab = jd.block_table;
  const int bsz = jd.block_size, bsh = jd.bs_shift, nblk = jd.n_blocks;

  // Operands of block c: B fragments, the lane's token scale and the block
  // table entries of the rows this lane stores (r = 8 it + lane / 8).
  uint4 Bn[KA];
  float Sn;
  int btn[4];
  auto fetch = [&](uint32_t c) {
    const uint8_t* blk = stg_job + (size_t)(tb0 + c) * BB;
#pragma unroll
    for (int s = 0; s < KS; ++s) Bn[s] = *(const uint4*)(blk + s * 1024 + lane * 16);
    // stage 1 writes no staging when no component is kept (KS == 0)
    Sn = KS > 0 ? *(const float*)(blk + KS * 1024 + (lane & 31) * 4) : 1.f;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint32_t tt = s1 + min(t0 + c * kDecTok + 8 * it + (lane >> 3), tc - 1);
      btn[it] = btab[bsh >= 0 ? tt >> bsh : tt / (uint32_t)bsz];
    }
  };
  // Operands in use: B fragments, token scale and the store addresses of
  // the lane's rows; taken over from the fetched ones only after the
  // block's stores were issued, so every wait covers loads alone.
  uint4 B[KA];
  float S;
  uint8_t* dp[4];
  auto take = [&](uint32_t c) {
#pragma unroll
    for (int s = 0; s < KS; ++s) B[s] = Bn[s];
    S = Sn;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint32_t tok = t0 + c * kDecTok + 8 * it + (lane >> 3);
      const uint32_t tt = s1 + tok;
      const int bt = btn[it];
      const bool blk_ok = bt >= 0 && bt < nblk;
      bad |= (int)(tok < tc && !blk_ok);
      const uint32_t in_blk = bsh >= 0 ? tt & ((1u << bsh) - 1u) : tt % (uint32_t)bsz;
      const long row = (long)bt * bsz + (long)in_blk;
      dp[it] = tok < tc && blk_ok ? dst + (row * F + f0) * OSZ + c16 * 16 : sink;
    }
  };
  if (c_lo + wave < c_hi) {
    fetch(c_lo + wave);
    take(c_lo + wave);
  }
  for (uint32_t c = c_lo + wave; c < c_hi; c += kGemmWaves) {
    fetch(min(c + kGemmWaves, c_hi - 1));   // unconditional: a fixed count of loads per block
    // Keep the scheduler from pulling the next block's takeover (which waits
    // for these loads) into this block's work.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
      const uint8_t* arow = As + (fb * 32 + (lane & 31)) * AST + 16 * h;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, *(const uint4*)(arow + 32 * s)),
                                                     __builtin_bit_cast(f16x8, B[s]), acc, 0, 0, 0);
      // D[feature][token]: token lane % 32, features 8 qd + 4 h + {0..3}
      uint8_t* srow = stg + (lane & 31) * kOutRow + (fb % BPS) * 32 * OSZ;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int fl = 8 * qd + 4 * h;
        const float4 m4 = *(const float4*)(mu_s + 32 * fb + fl);
        const float o0 = __builtin_fmaf(acc[4 * qd + 0], S, m4.x);
        const float o1 = __builtin_fmaf(acc[4 * qd + 1], S, m4.y);
        const float o2 = __builtin_fmaf(acc[4 * qd + 2], S, m4.z);
        const float o3 = __builtin_fmaf(acc[4 * qd + 3], S, m4.w);
        if (OUT32)
          *(float4*)(srow + fl * 4) = make_float4(o0, o1, o2, o3);
        else
          *(uint2*)(srow + fl * 2) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
      if (fb % BPS == BPS - 1) {
        const int fs = 32 * (fb - BPS + 1);            // segment's first feature in the slab
        const bool in_f = f0 + fs < F;                 // F % 64 == 0: whole segments
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint4 v = *(const uint4*)(stg + (8 * it + (lane >> 3)) * kOutRow + c16 * 16);
          // streaming (non-temporal) stores: the output is not read back here
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                      (u32x4*)(dp[it] == sink || !in_f ? sink : dp[it] + fs * OSZ));
        }
        wave_lds_sync();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    take(min(c + kGemmWaves, c_hi - 1));
  }
  if (bad) set_status(a, jd.status_idx, KVTC_E_INVALID);
  __syncthreads();  // the slab and staging rows are free for the next tile
}

// Stage 2 work is counted in units of one block of kDecTok tokens of one
// feature slab of one job, ordered (job, slab, block); job j's units start
// at tile_begin and number n_ctiles = slabs * blocks. The host launches at
// most as many workgroups as fit on the device at once and each takes an
// equal contiguous range of units, so all finish together; a range crosses
// few (job, slab) boundaries (the slab of V' is loaded once per segment),
// and the ranges in flight on one XCD cover the slabs of the same tokens.
template <int KS, bool OUT32>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void gemm_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint64_t U = a.total_tiles;
  const uint32_t g = logical_tile();
  uint32_t u = (uint32_t)(U * g / gridDim.x);
  const uint32_t u_end = (uint32_t)(U * (g + 1) / gridDim.x);
  while (u < u_end) {
    const int j = find_job(a, u);
    const JobDesc& jd = a.jobs[j];
    const uint32_t n_ch = (jd.tc + kDecTok - 1) / kDecTok;
    const uint32_t lu = u - jd.tile_begin;
    const uint32_t slab = lu / n_ch, c = lu - slab * n_ch;
    const uint32_t seg_end = min(u_end, jd.tile_begin + (slab + 1) * n_ch);
    gemm_segment<KS, OUT32>(a, j, slab, c, c + (seg_end - u), smem);
    u = seg_end;
  }
}

// Test hook: records -> codes (u8, one per component) and (shift, scale)
// pairs, the unpacking half of stage 1 on its own.
template <int G>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const LaunchArgs a, uint8_t* codes, float2* ssg) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const JobDesc& jd = a.jobs[0];
  CSlot& sl = slot_of(a, jd.slot);
  const uint32_t lt = tile - jd.tile_begin;
  if (lt >= jd.n_ctiles || sl.r_eff == 0) return;
  const uint32_t t0 = lt * kUnpackTile;
  const uint32_t n = min((uint32_t)kUnpackTile, jd.tc - t0);
  const int esz = a.dtype == KVTC_F32 ? 4 : 2;
  const int rb = sl.record_bytes;
  const uint8_t* recs = (const uint8_t*)jd.src + record_base(jd, a.F, esz) + (size_t)t0 * rb;
  stage_to_lds(smem, recs, (size_t)n * rb);
  __syncthreads();
  // One thread per (token, 8-component chunk).
  const int chunks = sl.r_eff / 8;
  for (int idx = threadIdx.x; idx < (int)n * chunks; idx += kThreads) {
    const int tl = idx / chunks, c = (idx % chunks) * 8;
    const uint8_t* rec = smem + (size_t)tl * rb;
    const int ag = c / G, o = c % G;
    *(uint64_t*)(codes + (size_t)(t0 + tl) * sl.r_eff + c) = get_codes8(rec, sl, ag, o);
    if (o == 0) {
      const uint64_t raw = lds_u64(rec + 8 * ag);
      ssg[(size_t)(t0 + tl) * sl.n_act + ag] =
          make_float2(__uint_as_float((uint32_t)raw), __uint_as_float((uint32_t)(raw >> 32)));
    }
  }
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
  CSlot& sl = slot_of(a, jd.slot);
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
  const int rbp = padded_stride(rb);
  if ((uint32_t)tl < n) {
    const uint32_t t = t0 + tl;
    for (int ag = 0; ag < sl.n_act; ++ag) {
      uint32_t cv[G / 2];
      for (int i = 0; i < G / 2; ++i) cv[i] = codes[(size_t)t * sl.r_eff + ag * G + h * (G / 2) + i];
      const float2 p = ss[(size_t)t * sl.n_act + ag];
      put_group<G>(smem + (size_t)tl * rbp, sl, ag, h, cv, p.x, p.y);
    }
  }
  __syncthreads();
  records_to_global((uint8_t*)jd.dst + record_base(jd, a.F, esz) + (size_t)t0 * rb, smem, n, rb, rbp);
}

// ------------------------------------------------------------- launchers ---

static dim3 grid_for(uint32_t tiles) { return dim3((tiles + 7u) / 8u * 8u); }

// Dynamic LDS above the 64 KiB default needs an explicit opt-in (gfx950 has
// 160 KiB per CU).
template <class K>
static void allow_lds(K kernel, size_t lds) {
  // a refusal surfaces as the launch error that follows
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Workgroups of `kernel` (threads, lds bytes) resident on the current
// device at once, at most max_per_cu per CU; a multiple of 8, at least 8.
template <class K>
static uint32_t resident_grid(K kernel, int threads, size_t lds, int max_per_cu = 1 << 20) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, threads, lds) != hipSuccess)
    return 8;
  const uint32_t n = (uint32_t)std::max(1, std::min(per_cu, max_per_cu)) * (uint32_t)std::max(1, cus);
  return std::max(8u, n / 8u * 8u);
}

// Optional cap on the persistent grids, encode and decode stage 2
// (environment variable KVTC_MAX_WORKGROUPS, rounded down to a multiple of
// 8, at least 8): fewer workgroups each walk more work. Unset or invalid:
// no cap.
static uint32_t persistent_grid_cap() {
  const char* e = std::getenv("KVTC_MAX_WORKGROUPS");
  if (!e || !*e) return UINT32_MAX;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (end == e || *end || v <= 0) return UINT32_MAX;
  return std::max<uint32_t>(8u, (uint32_t)std::min<long>(v, 1L << 20) / 8u * 8u);
}

// Encode workgroups per CU: the per-CU load throughput saturates at two
// (measured on llama31_8b, 32 tensors: 174 us per launch at one per CU,
// 143 at two, 150 at three).
constexpr int kEncMaxPerCU = 2;

template <int G, bool F32IN, bool ODD>
static int launch_encode_g(const LaunchArgs& a, int nb, size_t lds, hipStream_t s) {
  // Persistent: the resident workgroups (at most kEncMaxPerCU per CU), or
  // fewer when there are fewer compressed blocks (any grid covers the
  // headers and passthrough units).
#define KVTC_ENC(NBV)                                                                      \
  case NBV: {                                                                              \
    allow_lds(encode_kernel<NBV, G, F32IN, ODD>, lds);                                     \
    const dim3 g(std::min({grid_for(std::max(1u, (a.total_cblks + kEncWaves - 1) / kEncWaves)).x, \
                           resident_grid(encode_kernel<NBV, G, F32IN, ODD>, kThreads, lds,  \
                                         kEncMaxPerCU),                                    \
                           persistent_grid_cap()}));                                           \
    hipLaunchKernelGGL((encode_kernel<NBV, G, F32IN, ODD>), g, dim3(kThreads), lds, s, a); \
    break;                                                                                 \
  }
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
  const bool odd = (a.F / kEncKS) & 1;
#define KVTC_ENC_G(GV)                                                                   \
  if (G == GV)                                                                           \
    return f32 ? (odd ? launch_encode_g<GV, true, true>(a, nb, lds, s)                   \
                      : launch_encode_g<GV, true, false>(a, nb, lds, s))                 \
               : (odd ? launch_encode_g<GV, false, true>(a, nb, lds, s)                  \
                      : launch_encode_g<GV, false, false>(a, nb, lds, s));
  KVTC_ENC_G(16)
  KVTC_ENC_G(32)
#undef KVTC_ENC_G
  return (int)hipErrorInvalidValue;
}

// Decode launches take the exact K-step count ks = r_dec / 16 of every job
// in the batch (the host groups jobs by it).
#define KVTC_KS_CASES(X)                                                          \
  X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) \
  X(15) X(16)

int launch_prep(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  // one wave per compressed block; any grid covers the passthrough units
  const dim3 g = grid_for(std::max(8u, (a.total_tiles + kWaves - 1) / kWaves));
#define KVTC_PREP(KV)                                                       \
  case KV:                                                                  \
    allow_lds(prep_kernel<KV>, lds);                                        \
    hipLaunchKernelGGL((prep_kernel<KV>), g, dim3(kThreads), lds, s, a);    \
    break;
  switch (ks) {
    KVTC_KS_CASES(KVTC_PREP)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_PREP
  return (int)hipGetLastError();
}

template <bool OUT32>
static int launch_gemm_o(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
#define KVTC_GEMM(KV)                                                                        \
  case KV: {                                                                                 \
    allow_lds(gemm_kernel<KV, OUT32>, lds);                                                  \
    const dim3 g(std::min({std::max(8u, a.total_tiles / (8 * kGemmMinUnits) * 8),         \
                           resident_grid(gemm_kernel<KV, OUT32>, kGemmThreads, lds),       \
                           persistent_grid_cap()}));                                       \
    hipLaunchKernelGGL((gemm_kernel<KV, OUT32>), g, dim3(kGemmThreads), lds, s, a);              \
    break;                                                                                   \
  }
  switch (ks) {
    KVTC_KS_CASES(KVTC_GEMM)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_GEMM
  return (int)hipGetLastError();
}

int launch_gemm(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  return a.out_dtype == KVTC_F32 ? launch_gemm_o<true>(a, ks, lds, s) : launch_gemm_o<false>(a, ks, lds, s);
}

int launch_unpack(const LaunchArgs& a, int G, size_t lds, void* codes, void* ss, hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
  if (G == 16) {
    allow_lds(unpack_kernel<16>, lds);
    hipLaunchKernelGGL((unpack_kernel<16>), g, dim3(kThreads), lds, s, a, (uint8_t*)codes, (float2*)ss);
  } else if (G == 32) {
    allow_lds(unpack_kernel<32>, lds);
    hipLaunchKernelGGL((unpack_kernel<32>), g, dim3(kThreads), lds, s, a, (uint8_t*)codes, (float2*)ss);
  } else {
    return (int)hipErrorInvalidValue;
  }
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
