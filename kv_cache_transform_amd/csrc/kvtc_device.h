// Device-side helpers shared by the HIP translation units of libkvtc
// (kvtc_encode.hip, kvtc_decode.hip): vector types, conversions, device-state
// access, stream headers and status words, passthrough copies, and the
// record packing and unpacking routines that encode, decode and the test
// hooks all use. Also the host-side launch helpers common to every kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <utility>

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

// The last job whose first unit (JobDesc::tile_begin, or ::cblk_begin) is
// <= x: a binary search over the non-decreasing firsts, a chain of at most
// log2(kMaxLaunchJobs) + 1 uniform loads. A job with no units shares its first
// unit with the next job, so the search lands on the job that owns unit x.
template <uint32_t JobDesc::*M>
__device__ __forceinline__ int job_at(const LaunchArgs& a, uint32_t x) {
  int lo = 0, hi = a.n_jobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.jobs[mid].*M <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int find_job(const LaunchArgs& a, uint32_t tile) {
  return job_at<&JobDesc::tile_begin>(a, tile);
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

__device__ inline void write_header(const LaunchArgs& a, const JobDesc& jd, CSlot& sl) {
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
__device__ inline int check_header(const LaunchArgs& a, const JobDesc& jd, CSlot& sl) {
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
__device__ inline void encode_passthrough(const JobDesc& jd, uint32_t p, size_t row_bytes) {
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
__device__ inline bool decode_passthrough(const LaunchArgs& a, const JobDesc& jd, uint32_t p, long* rows_lds) {
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
__device__ inline void stage_to_lds(uint8_t* lds, const uint8_t* g, size_t n) {
  const size_t nv = n / 16;
  for (size_t i = threadIdx.x; i < nv; i += kThreads) ((uint4*)lds)[i] = ((const uint4*)g)[i];
  for (size_t i = nv * 16 + threadIdx.x; i < n; i += kThreads) lds[i] = g[i];
}

// Copy n bytes from LDS to 16-byte aligned global memory (cooperative).
__device__ inline void lds_to_global(uint8_t* g, const uint8_t* lds, size_t n) {
  const size_t nv = n / 16;
  for (size_t i = threadIdx.x; i < nv; i += kThreads) ((uint4*)g)[i] = ((const uint4*)lds)[i];
  for (size_t i = nv * 16 + threadIdx.x; i < n; i += kThreads) g[i] = lds[i];
}

// ------------------------------------------- record packing and unpacking ---
//
// The routines below are the only code that writes or reads the bits of a
// record; encode, decode and the kvtc_pack / kvtc_unpack test hooks all use
// them. Record layout: n_act (f32 shift, f32 scale) pairs, then each active
// group's chunk of G codes of its width w, code j at bits [j w, j w + w) of
// the chunk, least significant bit first.

// OR a run of four w-bit codes (packed LSB first in `run`, 4 w <= 32 bits)
// into a zeroed LDS record (as 32-bit words) at record bit `pos`: at most two
// words, with LDS atomics since the two half-waves' runs can share a word.
__device__ __forceinline__ void or_code_run(uint32_t* rw, uint32_t pos, uint32_t run, int w) {
  const uint32_t sh = pos & 31u;
  atomicOr(rw + (pos >> 5), run << sh);
  if (sh + 4u * (uint32_t)w > 32u) atomicOr(rw + (pos >> 5) + 1, run >> (32u - sh));
}

// One code of width w at record bit pos (a width per component): LDS words,
// atomics since neighbouring codes can share a word.
__device__ __forceinline__ void or_code(uint32_t* rw, uint32_t pos, uint32_t q, int w) {
  const uint32_t sh = pos & 31u;
  atomicOr(rw + (pos >> 5), q << sh);
  if (sh + (uint32_t)w > 32u) atomicOr(rw + (pos >> 5) + 1, q >> (32u - sh));
}

// Bit position in the record of component o of active group a (width w).
__device__ __forceinline__ uint32_t code_bit(CSlot& sl, int a, int o, int w) {
  return 8u * (uint32_t)slot_chunk(sl, a) + (uint32_t)(o * w);
}

// (shift, scale) of active group a into / out of a record (4-byte aligned
// for put_scales; any alignment for get_scales, see lds_u64).
__device__ __forceinline__ void put_scales(uint32_t* rw, int a, float shift, float scale) {
  rw[2 * a] = __float_as_uint(shift);
  rw[2 * a + 1] = __float_as_uint(scale);
}
__device__ __forceinline__ float2 get_scales(const uint8_t* rec, int a) {
  const uint64_t q = lds_u64(rec + 8 * a);
  return make_float2(__uint_as_float((uint32_t)q), __uint_as_float((uint32_t)(q >> 32)));
}

// The 64 record bits that start at the byte holding component o of active
// group a, where o is a multiple of 8 (so the 8 codes o .. o + 7 start on a
// byte boundary: 8 w bits).
__device__ __forceinline__ uint64_t code_bits8(const uint8_t* rec, CSlot& sl, int a, int o, int w) {
  return lds_u64(rec + slot_chunk(sl, a) + (o * w) / 8);
}

// The 8 codes of width W in the low 8 W bits of `bits`. The bit offsets are
// constants, so each code is one field extract (two where it straddles the
// 32-bit halves).
template <int W>
__device__ __forceinline__ void codes8_w(uint64_t bits, uint32_t (&v)[8]) {
  constexpr uint32_t mask = (1u << W) - 1u;
  const uint32_t lo = (uint32_t)bits, hi = (uint32_t)(bits >> 32);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j * W;
    if (p + W <= 32)
      v[j] = (lo >> p) & mask;
    else if (p >= 32)
      v[j] = (hi >> (p - 32)) & mask;
    else
      v[j] = __builtin_amdgcn_alignbit(hi, lo, p) & mask;
  }
}

// Copy n records of rb bytes from LDS rows of stride rbp into the contiguous
// stream at dst (16-byte aligned): 16-byte stores gathered from 4-byte (rb %
// 4 == 0) or 2-byte pieces, then a byte tail.
__device__ inline void records_to_global(uint8_t* dst, const uint8_t* lds, uint32_t n, int rb, int rbp) {
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


// Make this wave's LDS writes visible to its own lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until at most N vector memory operations of this wave are
// outstanding (s_waitcnt vmcnt(N); the other counters untouched). Memory
// operations complete in issue order for this count, so after it every one
// issued before the last N has completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N - 1, each call with its
// index as a compile-time constant (unrolling that does not depend on the
// optimizer's size limits: register arrays stay in registers).
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------ launch helpers ---

static inline dim3 grid_for(uint32_t tiles) { return dim3((tiles + 7u) / 8u * 8u); }

// Dynamic LDS above the 64 KiB default needs an explicit opt-in (gfx950 has
// 160 KiB per CU).
template <class K>
static inline void allow_lds(K kernel, size_t lds) {
  // a refusal surfaces as the launch error that follows
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Workgroups of `kernel` (threads, lds bytes) resident on the current
// device at once, at most max_per_cu per CU; a multiple of 8, at least 8.
template <class K>
static inline uint32_t resident_grid(K kernel, int threads, size_t lds, int max_per_cu = 1 << 20) {
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
static inline uint32_t persistent_grid_cap() {
  const char* e = std::getenv("KVTC_MAX_WORKGROUPS");
  if (!e || !*e) return UINT32_MAX;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (end == e || *end || v <= 0) return UINT32_MAX;
  return std::max<uint32_t>(8u, (uint32_t)std::min<long>(v, 1L << 20) / 8u * 8u);
}


}  // namespace kvtc
