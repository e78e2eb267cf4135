// Internal declarations shared by the host core (kvtc_host.cpp) and the HIP
// kernels and launchers (kvtc_encode.hip, kvtc_decode.hip). Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "kvtc.h"

namespace kvtc {

constexpr int kHeaderBytes = 64;
constexpr uint16_t kFormatVersion = 1;
constexpr int kScaleBits = 64;         // fp32 shift + fp32 scale per active group
constexpr int kMaxActGroups = 32;      // KVTC_MAX_REFF / smallest supported G (8)
constexpr int kMaxLaunchJobs = 32;     // jobs passed by value in one launch
constexpr size_t kAlign = 256;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Descriptor of one calibrated (layer, kind) inside the device state buffer.
// Offsets are bytes from the start of the device state.
struct alignas(16) DevSlot {
  uint64_t mu_off;        // f32 mu32[F]
  uint64_t venc_off;      // bf16 V'^T [r_enc][F]   (rows >= r_eff are zero)
  uint64_t vdec_off;      // f16  V'   F x r_dec in MFMA A-operand order (cols >= r_eff are zero)
  uint64_t mhi_off;       // f32  mu_hi[F] = bf16_rne(mu32), the encode's centring vector
  uint64_t cmu_off;       // f32  V'^T (mu32 - mu_hi) [r_enc], or V'^T mu32 when fold
                          // (rows >= r_eff are zero)
  uint64_t pcw_off;       // with a width per component: u32 [r_eff], per active component
                          // (bit position in the record << 8) | width
  uint64_t slot_id;
  int32_t calibrated;
  int32_t n_act;
  int32_t r_eff;
  int32_t record_bytes;
  int32_t r_enc;          // r_eff rounded up to 32 (encode MFMA blocks)
  int32_t r_dec;          // r_eff rounded up to 16 (decode MFMA K steps)
  int32_t G;
  int32_t F;
  int32_t pc;             // 1: a width per component (pcw_off), 0: a width per group
  int32_t fold;           // 1: the encode folds the mean into the product (cmu_off = V'^T mu32)
  uint8_t width[kMaxActGroups];        // width of active group a (its largest component's, pc)
  uint16_t chunk_off[kMaxActGroups];   // byte offset of its chunk in a record
};

// Per-job launch descriptor, passed by value in the kernel arguments.
struct JobDesc {
  const void* src;
  void* dst;
  const int32_t* block_table;
  const void* staging;     // decode stage 2 / stage-1 output
  uint32_t T;
  uint32_t s1;             // effective sink rows
  uint32_t w1;             // effective window rows
  uint32_t tc;             // compressed rows
  uint32_t tile_begin;     // first logical tile of this job
  uint32_t n_ctiles;       // compressed-row tiles
  uint32_t cblk_begin;     // encode: first 32-token block with records (jobs in order);
                           // decode stage 1: first header/passthrough unit
  int32_t slot;            // layer * 2 + kind
  int32_t layer;
  int32_t kind;
  int32_t block_size;      // paged output when block_table != nullptr
  int32_t n_blocks;
  int32_t status_idx;      // this job's word in LaunchArgs::status
  int32_t bs_shift;        // log2(block_size) if a power of two, else -1
};

struct LaunchArgs {
  JobDesc jobs[kMaxLaunchJobs];
  int32_t n_jobs;
  uint32_t total_tiles;
  int32_t dtype;           // stream / input element type
  int32_t out_dtype;       // decode output element type
  int32_t F;
  uint32_t total_cblks;    // encode: 32-token blocks with records; decode stage 1:
                           // header/passthrough units
  const uint8_t* state;    // device state base
  unsigned long long* status;  // per-launch slice of the workspace status words
  uint8_t* sink;           // kSinkBytes of workspace that absorb stores without a row
  uint32_t epoch;          // stamp of this launch (see status_word)
  int32_t pc;              // decode stage 1: every job's slot has a width per component
  int32_t fold;            // encode: every job's slot folds the mean into the product
  uint32_t wave_lds;       // decode stage 1: LDS bytes of each wave's record rows;
                           // fused decode: LDS bytes of each record buffer
};

// Workspace status words: (epoch << 32) | rank, combined with atomicMax so
// that every launch overrides older contents without a reset and the most
// severe result of a launch wins. Ranks: 0 OK, 1 INVALID (bad block table
// entry), 2 MISMATCH, 3 CORRUPT.
__host__ __device__ inline int status_rank(int st) {
  return st == KVTC_OK ? 0 : st == KVTC_E_INVALID ? 1 : st == KVTC_E_MISMATCH ? 2 : 3;
}
__host__ __device__ inline int rank_status(int rank) {
  return rank == 0 ? KVTC_OK : rank == 1 ? KVTC_E_INVALID : rank == 2 ? KVTC_E_MISMATCH : KVTC_E_CORRUPT;
}

// Tile sizes (tokens per workgroup tile).
constexpr int kEncTile = 128;
constexpr int kUnpackTile = 256;
constexpr int kPassRows = 16;
constexpr int kEncKS = 64;                 // features per LDS basis slice (encode)
constexpr int kEncRowPad = kEncKS + 8;     // bf16 elements per LDS basis row
constexpr int kEncBlk = 32;                // encode tokens per wave (one block)
constexpr int kEncWaves = kEncTile / kEncBlk;   // encode waves per tile

// Encode LDS: two basis slices [32 nb][kEncRowPad] bf16, then per wave its
// token tile of 32 rows of kEncKS raw input elements (padded by 16 bytes),
// then the centring vector mu_hi (F fp32). The centred token is split into
// enc_terms bf16 MFMA operands (two for bf16 input, three for f32).
__host__ __device__ constexpr int enc_terms(bool f32in) { return f32in ? 3 : 2; }
__host__ __device__ constexpr size_t enc_basis_bytes(int nb) { return (size_t)32 * nb * kEncRowPad * 2; }
__host__ __device__ constexpr int enc_xrow_bytes(bool f32in) { return kEncKS * (f32in ? 4 : 2) + 16; }
__host__ __device__ constexpr size_t enc_xtile_bytes(bool f32in) { return (size_t)32 * enc_xrow_bytes(f32in); }
__host__ __device__ constexpr size_t enc_lds_bytes(int nb, int F, bool f32in) {
  return 2 * enc_basis_bytes(nb) + kEncWaves * enc_xtile_bytes(f32in) + (size_t)F * 4;
}

// LDS row stride for records under assembly (encode, pack): a multiple of 4
// bytes with an odd dword count, so lanes of consecutive tokens write to
// different banks.
__host__ __device__ inline int padded_stride(int rb) {
  int p = (rb + 3) & ~3;
  if (((p >> 2) & 1) == 0) p += 4;
  return p;
}

// Decode. Stage 1 runs one wave per block of kDecTok compressed tokens and
// writes, per block, ks * 64 B-operand fragments of 16 bytes (fp16, MFMA
// lane order) and kDecTok f32 token scales: stg_block_bytes(ks) bytes. Its
// header and passthrough units cover kPrepPassRows rows each; the waves'
// record rows (stride dec_rec_stride(rb)) start at kPrepRowsOff of LDS.
constexpr int kDecTok = 32;
constexpr int kPrepPassRows = 4;
constexpr int kPrepWaves = 4;              // waves per stage-1 workgroup
constexpr int kPrepRowsOff = 64;           // after the passthrough row list (kPrepPassRows longs)
__host__ __device__ constexpr int dec_rec_stride(int rb) { return rb % 16 == 0 ? rb + 16 : rb; }
constexpr size_t kSinkBytes = 256;         // workspace target of stores that have no row
__host__ __device__ constexpr size_t stg_block_bytes(int ks) { return (size_t)ks * 1024 + kDecTok * 4; }

// Restore kernel (decode stage 2, and the whole decode when fused): units
// of one block of kDecTok compressed tokens of one slab of rest_slab(nfb)
// features of one job. kRestWaves waves, wave w owns 32 * nfb features of
// the slab with their V' fragments in registers; nfb = 4 needs ks <= 6 (the
// fragments and four accumulators then fit in 256 VGPRs) and F a multiple of
// 1024 (one slab covers 1024 features), else nfb = 2.
// LDS (bytes): the passthrough row list, the mu (fp32) of two slabs (the
// current segment's and the one before), the waves' output staging rows
// (kRestStgRow bytes each, 16-byte chunks XOR-swizzled by row), three
// fragment buffers (rest_frag_bytes: the B
// fragments and token scales of a block, then its 32 output rows as int32),
// and for the fused decode two record buffers of rec_lds bytes (32 record
// rows of stride dec_rec_stride(rb), 16 bytes of padding for 8-byte reads,
// then 32 int32 output rows).
constexpr int kRestWaves = 8;
constexpr int kRestThreads = 64 * kRestWaves;
constexpr int kRestPassRows = 8;
constexpr int kRestStgRow = 256;
__host__ __device__ constexpr int rest_nfb(int ks, int F) { return ks <= 6 && F % 1024 == 0 ? 4 : 2; }
__host__ __device__ constexpr int rest_slab(int nfb) { return kRestWaves * 32 * nfb; }
__host__ __device__ constexpr size_t rest_frag_bytes(int ks) { return stg_block_bytes(ks) + kDecTok * 4; }
// A batch's jobs share ks but not record_bytes; dec_rec_stride(rb) <= rb + 16
// <= rb_max + 16 bounds every job's row stride.
__host__ __device__ constexpr size_t rec_rows_bytes(int rb_max) { return (size_t)kDecTok * (rb_max + 16); }
__host__ __device__ constexpr size_t rest_rec_bytes(int rb_max) {
  return (rec_rows_bytes(rb_max) + 16 + 15) / 16 * 16 + kDecTok * 4;
}
constexpr size_t kRestMuOff = 64;
constexpr size_t kRestMuBytes = 4 * 1024;   // one slab's mu (rest_slab(4) floats)
constexpr size_t kRestStgOff = kRestMuOff + 2 * kRestMuBytes;
constexpr size_t kRestFragOff = kRestStgOff + (size_t)kRestWaves * kDecTok * kRestStgRow;
__host__ __device__ constexpr size_t rest_lds_bytes(int ks, bool fused, size_t rec_lds) {
  return kRestFragOff + 3 * rest_frag_bytes(ks) + (fused ? 2 * rec_lds : 0);
}

// ---------------------------------------------------------------------------
// Lossless stage: a KVTC stream <-> a KVTZ container (layout in kvtc.h at
// kvtc_lossless_encode). The stream is split into fields (passthrough byte
// planes, shift and scale byte planes, one field of codes per active group),
// each coded by static rANS in independent chunks of kLzChunk symbols, each
// chunk with kLzLanes interleaved states (one wavefront per chunk).
constexpr int kLzLanes = 64;
constexpr int kLzChunk = 256 * kLzLanes;
constexpr int kLzMBits = 12;
constexpr uint32_t kLzM = 1u << kLzMBits;
constexpr uint32_t kLzL = 1u << 16;
constexpr int kLzHead = 64;                 // container header, then the stream header
constexpr int kLzTables = kLzHead + kHeaderBytes;
constexpr int kLzMaxFields = 4 + 8 + kMaxActGroups;
constexpr int kLzPassBlk = 4096;            // passthrough elements per split/merge unit (16 a thread)
constexpr int kLzRecBlk = 64;               // records per split/merge unit
constexpr uint32_t kLzSeg = 16384;          // symbols per histogram unit
// record bytes: 8 per active group plus at most one per active component
constexpr int kLzMaxRec = 8 * kMaxActGroups + KVTC_MAX_REFF;

// The fields of one stream: esz passthrough planes of n_pt symbols, 4 shift
// and 4 scale planes of tc * n_act, then n_act code fields of tc * G.
struct LzShape {
  int esz, n_act, G;
  uint32_t n_pt, tc;
  const uint8_t* width;     // widths of the active groups, in order
};
__host__ __device__ inline int lz_nf(const LzShape& s) { return s.esz + 8 + s.n_act; }
__host__ __device__ inline uint32_t lz_n(const LzShape& s, int f) {
  return f < s.esz ? s.n_pt : f < s.esz + 8 ? s.tc * (uint32_t)s.n_act : s.tc * (uint32_t)s.G;
}
__host__ __device__ inline int lz_alpha(const LzShape& s, int f) {
  return f < s.esz + 8 ? 256 : 1 << s.width[f - s.esz - 8];
}
__host__ __device__ inline uint32_t lz_chunks(uint32_t n) { return (n + kLzChunk - 1) / kLzChunk; }
// a field's symbols in the workspace: 16-byte aligned, at least 16 bytes of
// padding behind them (whole 16-byte reads and 4-byte writes of a tail)
__host__ __device__ inline uint32_t lz_sym_region(uint32_t n) { return (n + 31) & ~15u; }

// Positions in the container and in a job's workspace region.
struct LzLayout {
  uint32_t n_chunks, n_segs;
  uint32_t dir_off, pay_off;        // container: chunk directory, payloads
  size_t sym, hist, fc, aux, cnt, state, dsto, scratch, bytes;   // workspace
};
// Field f's first symbol (workspace), first chunk, table entry (container)
// and first histogram unit, by prefix sums over the fields before it.
struct LzField {
  uint32_t sym_off, chunk0, tab_off, seg0;
};
__host__ __device__ inline LzField lz_field(const LzShape& s, int f) {
  LzField r = {0, 0, (uint32_t)kLzTables, 0};
  for (int g = 0; g < f; ++g) {
    const uint32_t n = lz_n(s, g);
    r.sym_off += lz_sym_region(n);
    r.chunk0 += lz_chunks(n);
    r.tab_off += 8 + 2 * (uint32_t)lz_alpha(s, g);
    r.seg0 += (n + kLzSeg - 1) / kLzSeg;
  }
  return r;
}
// encode: symbols, histograms, models (f | c << 16, then 1/f in fp64),
// per-chunk emitted-word counts, kLzLanes final states and payload offsets,
// and the scratch words; decode: symbols, then per field (kLzM words each)
// the symbol of every slot (kLzM bytes) and per symbol (f - 1) | c << 16.
__host__ __device__ inline LzLayout lz_layout(const LzShape& s, bool enc) {
  const int nf = lz_nf(s);
  const LzField e = lz_field(s, nf);
  LzLayout L;
  L.n_chunks = e.chunk0;
  L.n_segs = e.seg0;
  L.dir_off = e.tab_off;
  L.pay_off = (L.dir_off + 4 * L.n_chunks + 15) & ~15u;
  L.sym = 0;
  L.hist = align_up(e.sym_off, 256);
  L.fc = L.hist + (enc ? (size_t)nf * 256 * 4 : 0);
  L.aux = L.fc + (enc ? (size_t)nf * 256 * 4 : 0);
  L.cnt = align_up(L.aux + (size_t)nf * (enc ? 256 * 8 : kLzM * 4), 256);
  L.state = L.cnt + (size_t)L.n_chunks * 4;
  L.dsto = L.state + (size_t)L.n_chunks * 4 * kLzLanes;
  L.scratch = align_up(L.dsto + (size_t)L.n_chunks * 4, 256);
  L.bytes = align_up(L.scratch + (enc ? (size_t)L.n_chunks * kLzChunk * 2 : 0), 256);
  return L;
}
// Largest container a stream of this shape needs (one word per symbol, every
// chunk's kLzLanes states, and the 16-byte tail padding).
__host__ __device__ inline size_t lz_bound(const LzShape& s) {
  const LzLayout L = lz_layout(s, false);
  size_t b = L.pay_off + 15;
  for (int f = 0; f < lz_nf(s); ++f)
    b += 2 * (size_t)lz_n(s, f) + 4 * kLzLanes * (size_t)lz_chunks(lz_n(s, f));
  return b;
}

struct LzJob {
  const uint8_t* src;
  uint8_t* dst;
  uint8_t* ws;              // this job's workspace region (lz_layout)
  uint64_t src_cap;
  uint64_t stream_bytes;
  uint32_t T, s1, w1, tc;
  uint32_t unit0;           // first split/merge unit of the job in the launch
  uint32_t seg0;            // first histogram unit
  uint32_t field0;          // first field
  uint32_t chunk0;          // first chunk
  int32_t slot;
  int32_t status_idx;
};

struct LzArgs {
  LzJob jobs[kMaxLaunchJobs];
  int32_t n_jobs;
  int32_t esz;
  int32_t F;
  uint32_t units, segs, fields, chunks;   // totals of the launch
  uint32_t epoch;
  size_t rec_lds;                         // LDS bytes of one record block
  const uint8_t* state;
  unsigned long long* status;
  unsigned long long* sizes;              // container bytes per job (encode)
};

// Host-side launchers implemented in kvtc_encode.hip and kvtc_decode.hip (G = group size, lds =
// dynamic LDS bytes). Every job of one launch has the same shape parameter:
// nb = r_enc / 32 for encode, ks = r_dec / 16 for the decode stages. They
// return a hipError_t value cast to int.
int launch_encode(const LaunchArgs& a, int nb, int G, size_t lds, hipStream_t s);
int launch_prep(const LaunchArgs& a, int ks, size_t lds, hipStream_t s);
int launch_restore(const LaunchArgs& a, int ks, bool fused, size_t lds, hipStream_t s);
int launch_unpack(const LaunchArgs& a, int G, size_t lds, void* codes, void* ss, hipStream_t s);
// kvtc_decode_noalloc's workspace: this device's copy of a static device
// array (address looked up once per device), and its size.
int noalloc_scratch(void** ptr, size_t* bytes);
int launch_clear_words(void* words, int n, hipStream_t s);
int launch_status_codes(const void* words, int32_t* out, int n, hipStream_t s);
int launch_pack(const LaunchArgs& a, int G, size_t lds, const void* codes, const void* ss,
                hipStream_t s);
// kvtc_lossless.hip: the lossless stage's kernel sequences.
int launch_lz_encode(const LzArgs& a, hipStream_t s);
int launch_lz_decode(const LzArgs& a, hipStream_t s);

}  // namespace kvtc
