// attn_fwd.hip -- fused bf16 forward attention for MI355X (gfx950): without a
// mask or with a causal one, with as many K/V heads as query heads or fewer,
// over fixed-length or packed variable-length batches, with an optional
// per-row log-sum-exp.
//
// O = softmax(Q K^T / sqrt(128)) V per (batch, head, query row), the
// operation the snilld.dk page "Open source attention kernel in HIP beats
// AITER v3 on MI300X" describes (section "Hvordan kernen arbejder" / How the
// kernel works), streamed over key tiles with a running maximum and sum so
// the score matrix never leaves registers (the FlashAttention family the same
// page places the design in, section "Memory-placement og mikroarkitektur").
//
// Work decomposition.  One workgroup of 8 wave64s (two per SIMD) owns
// BM = 256 query rows of one (batch, head); each wave owns 32 of them.  Keys
// stream in tiles of BN = 64, shared through LDS by all eight waves.  Both
// products run on v_mfma_f32_32x32x16_bf16 in the transposed orientation
//     S^T (keys x queries)  = K   . Q^T      A = K tile (LDS), B = Q (VGPRs)
//     O^T (dims x queries) += V^T . P^T      A = V tile read transposed (LDS), B = P (VGPRs)
// so that every lane owns exactly one query row: the softmax row statistics
// are per-lane scalars plus one exchange between the two 32-lane halves, and
// the rescale of the output accumulator is a per-lane multiply.
//
// Split key ranges.  One workgroup runs per compute unit at a time, so when
// the (batch, head, q-tile) items do not fill the last round of compute units
// the items of that round can run as several workgroups over consecutive key
// ranges; each leaves unnormalised fp32 rows with their running maximum and
// sum, and attn_merge_kernel combines them (the same max-shifted sums as the
// online softmax) before the one rounding to bf16.  Under a causal mask this
// is done only when the items are nearly equal, each split item cutting its
// own visible tiles into equal ranges.
//
// Key shards.  The kPartial instantiation computes the rows over one shard
// of a head's keys (its causal diagonal given relative to the shard) and
// stores them in fp32, normalised by the shard's own sum, with the shard's
// log-sum-exp; attn_merge_shards_kernel combines shards by their
// log-sum-exps and rounds once: the per-device part of key parallelism.
//
// Extensions the pages list as missing from the kernel they describe (their
// section "Hvad er udgivet" / What was released): a causal mask (CAUSAL: the
// tiles past a row's limit are never visited, the diagonal ones are masked
// beside the row maxima), grouped K/V heads (query head h reads K/V head
// h / kv_group) and packed variable-length batches (VARLEN: each sequence's
// offsets read on the device).  The per-row log-sum-exp comes from the same
// running maximum and sum as the output.
//
// MFMA 32x32x16 operand layout (lane l, g = l / 32):
//     A[i][k]: lane supplies row i = l % 32, k = 8g .. 8g+7
//     B[k][j]: lane supplies column j = l % 32, k = 8g .. 8g+7
//     C[i][j]: lane holds column j = l % 32, rows 8r + 4g + t in element 4r + t
//
// Data movement.  K and V tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (lane l of a load lands at 16*l past the
// wave's LDS base), four stages deep with loads issued three tiles ahead,
// one workgroup barrier per tile.  The buffer descriptor of each tile ends at
// the last valid key, so keys past Sk read as zeros without any per-lane
// test, and past the last tile the range is empty, so every iteration issues
// the same loads and waits.  LDS rows are 256 bytes, with the 16-byte chunks
// XOR-swizzled by row so the MFMA operand reads are free of bank conflicts
// on gfx950's 64-bank LDS (16 lanes per cycle for 16-byte reads, 32 lanes
// per cycle for 8-byte reads): K chunk c of row r sits at c ^ (r % 16), V
// chunk c of row r at c ^ 4(r % 4).
//
// Schedule.  Each wave software-pipelines its tiles: iteration t computes
// the K.Q logits of tile t+1 on the matrix core while the VALU turns the
// logits of tile t into weights (exp2, row sum, bf16 pack), then the P.V
// product of tile t while the VALU reduces the row maxima of tile t+1.  The
// loads of tile t+3 are issued one instruction at a time between MFMAs.
// Without a causal mask, when Sk is not a multiple of 64 the ragged last key
// tile is visited first, so the one key mask happens before the loop.
//
// Key order inside a 32-key block.  LDS K row i holds key
// pi(i) = 16*(i/4 % 2) + 4*(i/8) + i%4, so that after the first product lane
// group g holds the 16 consecutive keys 16g .. 16g+15 of the block in
// elements 0..15.  Eight of those are exactly a B operand of the second
// product; the matching A operand (8 consecutive keys of one V column) comes
// from two ds_read_b64_tr_b16 reads of the row-major V tile.  Within each
// 16-lane group that instruction hands lane i element i%4 of the 8-byte
// chunks addressed by lanes 4s + i/4 (s = 0..3); pointing lane 4s + u at keys
// key0 + s, dims dim0 + 4u .. 4u+3 gives lane i the four keys key0 .. key0+3
// at dim dim0 + i.
//
// Numerics.  Logits accumulate in fp32 on the matrix cores.  The softmax runs
// in the base-2 domain: t = s * log2(e)/sqrt(128) (one fp32 constant), the
// running maximum m starts at -FLT_MAX (finite, so an all -Inf prefix never
// forms -Inf - -Inf) and is kept rounded up so the maximal key's weight is
// never above 1, p = exp2(t - m) on the hardware exp, the row sum l in fp32
// from the unrounded p.  The maximum (and with it the accumulator) is only
// moved when some row's maximum grew by more than 2^8: between moves the
// weights stay below 256, which fp32 and bf16 carry without loss of relative
// precision.  P is rounded to bf16 (nearest-even) for the second product.
// The epilogue multiplies by 1/l and rounds once to bf16 in the requested
// mode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "attn_fwd.h"

namespace {

constexpr int D = 128;
constexpr int BM = 256;                // query rows per workgroup
constexpr int BN = 64;                 // keys per tile
constexpr int kPartial = 3;            // MODE of the instantiation that stores fp32 rows of one key shard
// The tile loads address the 64 K/V rows of a tile with 32-bit buffer
// offsets: 63 row strides + 256 bytes must stay below 2^32.  The row stride is
// H_kv * 256 bytes in BSHD and packed layouts, so H_kv (and H >= H_kv) is
// capped at 2^18: 63 * 2^26 + 256 < 2^32.
constexpr int64_t kMaxHeads = int64_t(1) << 18;
constexpr int NWAVES = BM / 32;        // 32 query rows per wave: 8 waves, two per SIMD
constexpr int NTHREADS = NWAVES * 64;
constexpr int TILE_BYTES = BN * D * 2; // one K or V tile in LDS (16 KiB)
constexpr int NSTAGE = 4;              // LDS stages: tiles are loaded three ahead
constexpr float kRescaleLog2 = 8.0f;   // move the running maximum only past 2^8

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// the next tile's loads are issued one at a time after these MFMAs of each
// half of an iteration
constexpr int kHookAt0 = 1, kHookAt1 = 9;
// log2(e) / sqrt(128), rounded to fp32
constexpr float kScaleLog2 = 0.12751743082459868f;
// 1 / kScaleLog2, rounded to fp32: turns a threshold on scaled logits into one on raw logits
constexpr float kInvScaleLog2 = 7.84206485748291f;
// gfx9 buffer descriptor word 3: 32-bit data format, no swizzle, raw addressing
constexpr int kBufferWord3 = 0x00020000;

struct Geometry {
  int64_t q_row;   // element stride between consecutive query rows
  int64_t k_row;   // element stride between consecutive key rows
  int64_t q_head;  // element offset of head h within batch b: q_head * h
  int64_t k_head;
  int64_t q_batch; // element offset of batch b
  int64_t k_batch;
  int64_t kv_group; // query heads per K/V head: query head h reads K/V head h / kv_group
};

// Work items are (b, h, q-tile) in row-major order.  Items [0, n_whole) run
// whole, one workgroup each; every later item runs as `splits` workgroups,
// each over `tiles_per_split` consecutive key tiles of the visiting order,
// leaving its unnormalised output rows (fp32), the running maximum m (base-2
// scaled logits) and row sum l of its key range in the workspace for
// attn_merge_kernel.  Partial slot r (= workgroup id - n_whole) holds
//     part[(r * BM + row) * D + c],  ml[(r * BM + row) * 2 + {0: m, 1: l}].
struct Split {
  int n_whole;
  int splits;
  int tiles_per_split;
  float* part;
  float* ml;
  // 0: the split items are work items n_whole, n_whole + 1, ... in order.
  // Otherwise every item is split (n_whole = 0) and this is the number of
  // (b, h) pairs: split item i is q-tile rank i / qt_major of pair
  // i % qt_major, so the longest q-tiles of every head come first.
  int qt_major;
};

// work item (b, h, q-tile rank) of split item i
__device__ __forceinline__ int split_item_work(const Split& sp, int i, int n_qtiles) {
  return sp.qt_major ? (i % sp.qt_major) * n_qtiles + i / sp.qt_major : sp.n_whole + i;
}

// Variable-length batches: sequence b holds the packed query rows
// cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1 (offsets read on
// the device, clamped to [0, total] so that no access leaves the tensors
// whatever they hold).
struct Varlen {
  const int* cu_q;
  const int* cu_k;
  int total_q;
  int total_k;
  int n_groups;  // B * H_kv: (sequence, K/V head) groups
};

// Combine a per-lane value with the one held 32 lanes away (the other half of
// the wave).  This goes through ds_bpermute: AMD clang 22 folds
// fmaxf(r[0], r[1]) of __builtin_amdgcn_permlane32_swap(x, x) into r[0], as
// if the swap of a register with itself were the identity, which leaves the
// two halves with different values (a swap whose second operand is hidden
// from the compiler is correct but measured no faster here).
__device__ __forceinline__ float wave_half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
// fp32 addition is commutative, so both halves get identical bits
__device__ __forceinline__ float wave_half_sum(float x) { return x + __shfl_xor(x, 32); }

template <int MODE>
__device__ __forceinline__ uint16_t round_to_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (MODE == ATTN_ROUND_RTNE) {
    __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: nearest-even, NaN stays NaN
    return __builtin_bit_cast(uint16_t, b);
  }
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN: canonical quiet NaN
  if (MODE == ATTN_ROUND_RTNA) return (uint16_t)((u + 0x8000u) >> 16);
  return (uint16_t)(u >> 16);  // RTZ
}

// pi within a 32-key block: LDS row -> key
__device__ __forceinline__ int key_of_k_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: 48-bit base, stride 0, num_records bytes, word 3.
// All four words are wave-uniform (scalar registers).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)num_records);
  r[3] = kBufferWord3;
  return r;
}

// One direct-to-LDS load: 16 bytes per lane from rsrc + voffset land at
// lds_base + 16 * lane.  Written as a single-instruction asm wrapper (plus
// the one-cycle M0 hazard wait) so the compiler does not
// track it as an LDS write: it would otherwise wait for every such load in
// flight before each later LDS read, since it cannot tell which stage a load
// fills.  The kernel orders these loads itself with s_waitcnt vmcnt and the
// workgroup barrier (loads complete in order).  The LDS address goes in
// through an M0 operand, so the compiler writes M0 itself and knows it is
// taken; the s_nop covers the one wait state between that write and the load.
__device__ __forceinline__ void lds_dma_b128(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "{m0}"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory");
}

// LDS address (offset within the workgroup's LDS) of a __shared__ pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// SPLIT: the grid may hold split work items (sp describes them); without it
// every workgroup runs one whole item and the key range is known statically.
// VARLEN (not with SPLIT): the items are (sequence, head, q-tile) of a packed
// variable-length batch; Sq and Sk are the sequence's own, and items past a
// sequence's last q-tile exit at once.
// CAUSAL: query row r attends to the keys
// j <= min(r + causal_off, Sk - 1) only: causal_off_fixed (the host's 0, Sk - Sq,
// or a key shard's offset from the global diagonal), or with VARLEN 0 or the
// sequence's Sk - Sq (causal_br).  The workgroup visits the key tiles
// 0 .. up to its last row's limit in order (so the q-tiles of a head stream
// the same tiles together, as without a mask): those every row sees whole in
// a loop without mask code, then the diagonal ones (some row's limit falls
// inside or before them) with the mask applied beside the row maxima; a wave
// past the last tile its own rows see only loads and meets the barriers.
// With SPLIT, a split item's visible tiles are cut into sp.splits ranges of
// equal length (the last ones may be shorter or empty).
// In every instantiation a wave whose 32 rows all lie past Sq (the ragged
// last q-tile) skips the products and only loads.
template <int MODE, bool SPLIT, bool CAUSAL, bool VARLEN>
__device__ __forceinline__ void attn_item(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O, int H,
                                          int Sq_all, int Sk_all, int n_qtiles, const Geometry& g, const Split& sp,
                                          const Varlen& vl, int causal_br, int64_t causal_off_fixed,
                                          float* __restrict__ lse, uint8_t* lds, int work, int t_begin, int t_end,
                                          int slot) {
  // K stages in the lower 64 KiB, V stages in the upper 64 KiB
  uint8_t* const k_st[NSTAGE] = {lds, lds + TILE_BYTES, lds + 2 * TILE_BYTES, lds + 3 * TILE_BYTES};
  uint8_t* const v_st[NSTAGE] = {lds + 4 * TILE_BYTES, lds + 5 * TILE_BYTES, lds + 6 * TILE_BYTES,
                                 lds + 7 * TILE_BYTES};
  const int id = blockIdx.x;
  // causal: a head's q-tiles in decreasing order, the ones with the most
  // visible keys dispatched first
  int qt = CAUSAL ? n_qtiles - 1 - work % n_qtiles : work % n_qtiles;
  int h = (work / n_qtiles) % H, b = work / n_qtiles / H;
  if constexpr (VARLEN) {
    // Sequences differ in length, so contiguous item ranges per XCD would
    // load them unevenly.  Instead the (sequence, K/V head) groups are dealt
    // to the XCDs in turn (with H_kv = 8 every XCD gets one K/V head of every
    // sequence); a group's items (its query heads x q-tiles, the heads of one
    // q-tile together) stay on one XCD and share that K/V head in its L2.
    const int hpg = (int)g.kv_group, gitems = hpg * n_qtiles;
    const int xcd = id & 7, local = id >> 3;
    const int group = xcd + 8 * (local / gitems), r = local % gitems;
    if (group >= vl.n_groups) return;
    const int H_kv = H / hpg;
    b = group / H_kv;
    h = (group % H_kv) * hpg + r % hpg;
    qt = CAUSAL ? n_qtiles - 1 - r / hpg : r / hpg;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  // this item's sequence: its lengths and the element offsets of its first
  // query and key rows (batch b of the tensors, or packed rows with VARLEN)
  int Sq = Sq_all, Sk = Sk_all;
  int64_t q_base = b * g.q_batch, k_base = b * g.k_batch;
  // log-sum-exp of query row i of this item: lse[lse_row0 + i], laid out
  // [B, H, Sq] (VARLEN: [H, total_q])
  int64_t lse_row0 = ((int64_t)b * H + h) * Sq_all;
  if constexpr (VARLEN) {
    const int q0 = min(max(vl.cu_q[b], 0), vl.total_q), q1 = min(max(vl.cu_q[b + 1], q0), vl.total_q);
    const int k0 = min(max(vl.cu_k[b], 0), vl.total_k), k1 = min(max(vl.cu_k[b + 1], k0), vl.total_k);
    Sq = q1 - q0;
    Sk = k1 - k0;
    q_base = (int64_t)q0 * g.q_row;
    k_base = (int64_t)k0 * g.k_row;
    lse_row0 = (int64_t)h * vl.total_q + q0;
    if (qt * BM >= Sq) return;  // past the sequence's last q-tile (the whole workgroup leaves)
  }
  const int n_tiles_all = (Sk + BN - 1) / BN;
  const int64_t causal_off = VARLEN ? (causal_br ? Sk - Sq : 0) : causal_off_fixed;
  const uint16_t* Qh = Q + q_base + h * g.q_head;
  // (the integer division runs on the vector unit; made uniform again so that
  // the K/V pointers, and the per-tile addresses formed from them, stay scalar)
  const int hk = __builtin_amdgcn_readfirstlane(h / (int)g.kv_group);
  const uint16_t* Kh = K + k_base + hk * g.k_head;
  const uint16_t* Vh = V + k_base + hk * g.k_head;
  uint16_t* Oh = O + q_base + h * g.q_head;
  if (VARLEN && Sk == 0) {
    // a sequence without keys: the 0/0 of an empty softmax, NaN rows; the
    // log of an empty sum, -Inf
    const int row = qt * BM + (int)(threadIdx.x >> 6) * 32 + (threadIdx.x & 31);
    if (row < Sq) {
      const int half = (threadIdx.x >> 5) & 1;
      uint16_t* dst = Oh + (int64_t)row * g.q_row + 64 * half;
#pragma unroll
      for (int i = 0; i < 8; ++i) *(u32x4*)(dst + 8 * i) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
      if (lse && half == 0) lse[lse_row0 + row] = -__builtin_inff();
    }
    return;
  }
  const uint32_t row_bytes = (uint32_t)(g.k_row * 2);

  // ---- Q fragments: this lane's query row, dims 16ks + 8grp .. +7 ----
  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8 qf[8];
  {
    const bool ok = qrow < Sq;
    const uint16_t* src = Qh + (int64_t)(ok ? qrow : 0) * g.q_row + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 w = ok ? *(const u32x4*)(src + 16 * ks) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // Q must be in registers before the tile loop: the compiler cannot see the
  // direct-to-LDS loads and would otherwise re-wait for Q inside the loop,
  // draining the tile loads in flight with it.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- direct-to-LDS load assignment: wave w issues loads j = 2w + u ----
  // Load j fills LDS rows 4j .. 4j+3 (1 KiB); lane l writes row 4j + l/16 at
  // 16-byte position l%16, which holds logical chunk (l%16) ^ swizzle(row).
  uint32_t k_src[2], v_src[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 4 * (2 * wave + u) + (lane >> 4);
    const int p = lane & 15;
    const int kc = p ^ (r & 15);
    const int key = (r & 32) + key_of_k_row(r & 31);
    k_src[u] = (uint32_t)key * row_bytes + 16u * kc;
    const int vc = p ^ (4 * (r & 3));
    v_src[u] = (uint32_t)r * row_bytes + 16u * vc;
  }

  // ---- MFMA operand read offsets (bytes within a tile) ----
  // K: row l32 (+32 kb), logical chunk 2ks + grp at position chunk ^ (row % 16)
  uint32_t k_rd[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_rd[ks] = 256u * l32 + 16u * ((2 * ks + grp) ^ (l32 & 15));
  // V (transposed reads): lane 16G + 4s + u reads keys 16(G/2) + 4half + s
  // (+32kb + 8hh), dims 32db + 16(G%2) + 4u .. +3, logical chunk
  // 4db + 2(G%2) + u/2 at position chunk ^ (4 * (row % 4))
  uint32_t v_rd[4][2];
  {
    const int G = lane >> 4, sidx = (lane >> 2) & 3, u4 = lane & 3;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = 16 * (G >> 1) + 4 * half + sidx;
        const int chunk = 4 * db + 2 * (G & 1) + (u4 >> 1);
        v_rd[db][half] = 256u * row + 16u * (chunk ^ (4 * (row & 3))) + 8u * (u4 & 1);
      }
  }

  // The same offsets as LDS addresses in V stage 0, hidden from the compiler so
  // that it keeps them in registers and folds the stage and block offsets
  // (below 64 KiB) into each read's immediate offset field.
  lds_u8_t* v_rd_lds[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t a = lds_addr(v_st[0]) + v_rd[db][half];
      asm volatile("" : "+v"(a));
      v_rd_lds[db][half] = (lds_u8_t*)(uintptr_t)a;
    }

  // Key tiles are visited in the order n-1, 0, 1, ..., n-2 when the last one
  // is ragged, so that the only tile that needs a key mask is the first one,
  // handled before the main loop (the order of the online softmax updates is
  // free; only rounding depends on it).  Otherwise in the order 0 .. n-1.
  // This workgroup visits positions t_begin .. t_end-1 of that order; loop
  // indices below count from t_begin.
  int n_tiles = SPLIT ? t_end - t_begin : n_tiles_all;
  const bool ragged = (Sk % BN) != 0;
  // CAUSAL: this lane's last visible key (negative: none); the number of key
  // tiles the workgroup visits, up to its last row's limit (at least one:
  // when no row sees a key, tile 0 is visited fully masked, l stays 0 and
  // every row ends as 0 * (1/0) = NaN); the first diagonal tile diag0 (the
  // first row's limit falls inside it: every earlier tile is visible to all
  // rows).
  int row_lim = 0, diag0 = 0;
  if constexpr (CAUSAL) {
    const int64_t last_key = (int64_t)Sk - 1;
    const int64_t lim = (int64_t)qrow + causal_off;
    row_lim = (int)(lim < last_key ? (lim < -1 ? -1 : lim) : last_key);  // -1: no key
    const int64_t r_last = ((int64_t)qt * BM + BM < Sq ? (int64_t)qt * BM + BM : (int64_t)Sq) - 1;
    const int64_t hi = r_last + causal_off < last_key ? r_last + causal_off : last_key;
    n_tiles = hi < 0 ? 1 : (int)(hi / BN) + 1;
    const int64_t r0 = (int64_t)qt * BM + causal_off;
    const int64_t lo = r0 < last_key ? r0 : last_key;
    diag0 = lo < 0 ? 0 : (int)((lo + 1) / BN);
    if (SPLIT && slot >= 0) {
      // this workgroup's share of the item's visible tiles
      const int per = (n_tiles + sp.splits - 1) / sp.splits;
      t_begin = (slot % sp.splits) * per;
      t_end = t_begin + per < n_tiles ? t_begin + per : n_tiles;
      n_tiles = t_end - t_begin;
      if (n_tiles <= 0) {
        // an empty range: the partial of no keys (m = -FLT_MAX, l = 0, rows
        // 0), which the merge weighs with 0 (or, when no range saw a key,
        // turns into the 0 * (1/0) = NaN of a row without keys)
        const int row = wave * 32 + l32;
        float* prow = sp.part + ((int64_t)slot * BM + row) * D + 4 * grp;
#pragma unroll
        for (int i = 0; i < 16; ++i) *(f32x4*)(prow + 8 * i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (grp == 0) *(f32x2*)(sp.ml + ((int64_t)slot * BM + row) * 2) = f32x2{-3.402823466e38f, 0.0f};
        return;
      }
    }
  }
  // Buffer resources of the K and V rows of the seq-th visited tile.  Past
  // the last tile the range is empty: those loads touch no memory (the
  // hardware range check turns them into zeros), so every iteration issues
  // the same number of loads and the load-count waits need no branches.
  auto tile_rsrc = [&](int t, i32x4& rk, i32x4& rv) __attribute__((always_inline)) {
    const int seq = SPLIT ? t_begin + t : t;
    const int tile = CAUSAL || !ragged ? seq : (seq == 0 ? n_tiles_all - 1 : seq - 1);
    const bool live = t < n_tiles;
    const int base = live ? tile * BN : 0;
    const int valid = Sk - base < BN ? Sk - base : BN;
    const uint32_t nrec = live ? (uint32_t)(valid - 1) * row_bytes + 256u : 0u;
    rk = make_rsrc(Kh + (int64_t)base * g.k_row, nrec);
    rv = make_rsrc(Vh + (int64_t)base * g.k_row, nrec);
  };
  // this wave's two 1 KiB pieces of a K (or V) tile of LDS stage `stage`,
  // straight into LDS.  `lw` is the wave's LDS base (its pieces start 2 KiB
  // apart); the loop passes it through an empty asm each iteration so that the
  // compiler adds the stage offsets where they are used instead of keeping
  // sixteen precomputed addresses in scalar registers across the loop.
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(lds) + 2048u * (uint32_t)wave);
  auto dma_k = [&](const i32x4& rk, uint32_t lw, int stage, int u) __attribute__((always_inline)) {
    lds_dma_b128(rk, lw + (uint32_t)(stage * TILE_BYTES + 1024 * u), k_src[u]);
  };
  auto dma_v = [&](const i32x4& rv, uint32_t lw, int stage, int u) __attribute__((always_inline)) {
    lds_dma_b128(rv, lw + (uint32_t)((NSTAGE + stage) * TILE_BYTES + 1024 * u), v_src[u]);
  };
  auto issue_loads = [&](int seq, int stage) __attribute__((always_inline)) {
    i32x4 rk, rv;
    tile_rsrc(seq, rk, rv);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      dma_k(rk, lds_wave, stage, u);
      dma_v(rv, lds_wave, stage, u);
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = -3.402823466e38f;
  float l_run = 0.0f;
  // the raw logit past which the running maximum moves: (m_run + 8) / c in
  // fp32, kept with m_run (-Inf while m_run is -FLT_MAX: any finite logit
  // moves it then)
  float m_thr = -__builtin_inff();

  f32x16 S[2][2];      // logits of two tiles: the one being turned into weights, the next one
  bf16x8 pf[2][2];     // weights of the current tile, the B operand of P.V
  float mx = 0.0f;     // maximum of the next tile's logits over this lane's half of the row

  // S^T = K . Q^T for the two 32-key blocks of one tile (K stage kt)
  auto qk = [&](f32x16 (&s)[2], const uint8_t* kt) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kt + k_rd[ks] + 8192 * kb);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
  };
  // keys past Sk of key tile `tile` get a -Inf logit
  auto mask_tail = [&](f32x16 (&s)[2], int tile) __attribute__((always_inline)) {
    const int base = tile * BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < 16; ++n)
        if (base + 32 * kb + 16 * grp + n >= Sk) s[kb][n] = -__builtin_inff();
  };
  // CAUSAL: keys past this lane's limit in key tile `tile` get a -Inf logit
  // (element n of block kb holds key 64 tile + 32kb + 16grp + n)
  auto mask_causal = [&](f32x16 (&s)[2], int tile) __attribute__((always_inline)) {
    const int rel = row_lim - tile * BN - 16 * grp;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < 16; ++n)
        if (32 * kb + n > rel) s[kb][n] = -__builtin_inff();
  };
  // (the reductions start from -Inf, which fmaxf drops, so that they are all
  // v_max3: starting from the first logit made this compiler quiet the first
  // two logits with v_max x,x and pair them with a third v_max.  A half row
  // of NaN or -Inf logits now gives -Inf where it gave NaN; both compare
  // false in the rescale test and drop out of a move.)
  auto rowmax = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) {
    float m = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < 16; ++n) m = fmaxf(m, s[kb][n]);
    mx = m;
  };
  // Move the running maximum when some row's maximum grew past 2^8 above it:
  // one compare of the raw maximum against m_thr per tile (m_thr carries the
  // fp32 rounding of (m + 8) / c, so a maximum within a few ulp of the
  // threshold may stay, and its weight reach 2^8 times 1 + a few ulp).
  // Whether any row grew is decided from each lane's half of its row (a
  // row's maximum grew past the threshold iff one of its halves did), so the
  // exchange between the two halves is only needed on the rare move itself.
  // The candidate is the scaled row maximum rounded up by at least half an
  // ulp: then fma(s, c, -m) <= 0 for the maximal logit, its weight
  // exp2(<= 0) <= 1 rounds to exactly 1 in bf16, so a row dominated by one
  // key (or with a single key) returns that V row exactly in every mode.
  // (-Inf and NaN maxima compare false; in a move, fmaxf ignores a NaN half.)
  auto rescale = [&]() __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(mx > m_thr) != 0) {
      const float mr = wave_half_max(mx) * kScaleLog2;
      const float m_new = fmaxf(m_run, __builtin_fmaf(__builtin_fabsf(mr), 0x1p-23f, mr));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      m_thr = (m_run + kRescaleLog2) * kInvScaleLog2;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    }
  };

  // weights 2i and 2i+1 of the current tile (logits sc) into the bf16 operand
  // of P.V, their sum into psum
  auto weight_pair = [&](const f32x16 (&sc)[2], int i, float& psum) __attribute__((always_inline)) {
    const int kb = i >> 3, hh = (i >> 2) & 1, q2 = i & 3, n = 8 * hh + 2 * q2;
    f32x2 p;
    p[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][n], kScaleLog2, -m_run));
    p[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][n + 1], kScaleLog2, -m_run));
    // (weights are >= +0, so starting from the first one equals 0 + it)
    psum = i == 0 ? p[0] : psum + p[0];
    psum += p[1];
    const bf16x2 pb = __builtin_convertvector(p, bf16x2);
    pf[kb][hh][2 * q2] = pb[0];
    pf[kb][hh][2 * q2 + 1] = pb[1];
  };
  // Region A: K.Q of the next tile (sn, K stage kt) interleaved with the
  // weights of the current one (sc): one MFMA, then one pair of weights.
  // K operands are read four MFMAs ahead.
  auto qk_weights = [&](f32x16 (&sn)[2], const f32x16 (&sc)[2], const uint8_t* kt, auto&& hook)
                        __attribute__((always_inline)) {
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    bf16x8 ka[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = *(const bf16x8*)(kt + k_rd[i >> 1] + 8192 * (i & 1));
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 4 < 16) ka[i + 4] = *(const bf16x8*)(kt + k_rd[(i + 4) >> 1] + 8192 * ((i + 4) & 1));
      sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[i >> 1], sn[i & 1], 0, 0, 0);
      if (i == kHookAt0) hook(0);
      if (i == kHookAt1) hook(1);
      weight_pair(sc, i, psum);
    }
    l_run += psum;
  };
  // the weights of a wave's last tile, with no next tile to compute
  auto weights = [&](const f32x16 (&sc)[2]) __attribute__((always_inline)) {
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) weight_pair(sc, i, psum);
    l_run += psum;
  };
  // the V operand of P.V MFMA i (keys 32kb + 8hh.., dims 32db..) from V stage vstage
  auto v_operand = [&](int vstage, int i) __attribute__((always_inline)) {
    const int kb = i >> 3, hh = (i >> 2) & 1, db = i & 3;
    const int off = vstage * TILE_BYTES + 256 * (32 * kb + 8 * hh);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(v_rd_lds[db][0] + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(v_rd_lds[db][1] + off));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Region B: P.V of the current tile (V stage vt) interleaved with the row
  // maxima of the next tile's logits: one MFMA, then two maxima.
  // MASKED: the logits of key tile `ntile` get the causal mask first (keys
  // past the lane's limit become -Inf), two per MFMA like the maxima
  auto pv_rowmax = [&](auto masked_c, int vstage, f32x16 (&sn)[2], int ntile, auto&& hook)
                       __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int rel = row_lim - ntile * BN - 16 * grp;
    bf16x8 va[16];
    auto vread = [&](int i) __attribute__((always_inline)) { va[i] = v_operand(vstage, i); };
#pragma unroll
    for (int i = 0; i < 4; ++i) vread(i);
    float m = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 4 < 16) vread(i + 4);
      const int kb = i >> 3, hh = (i >> 2) & 1, db = i & 3;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pf[kb][hh], acc[db], 0, 0, 0);
      if (i == kHookAt0) hook(0);
      if (i == kHookAt1) hook(1);
      {
        // (a select into a temporary written back whole: the same mask as a
        // conditional store into the accumulator made this compiler emit about
        // 270 selects per tile instead of 32, and use 102 scalar registers)
        const int n = 2 * (i & 7), key = 32 * (i >> 3) + n;
        float x0 = sn[i >> 3][n], x1 = sn[i >> 3][n + 1];
        if (MASKED) {
          x0 = key > rel ? -__builtin_inff() : x0;
          x1 = key + 1 > rel ? -__builtin_inff() : x1;
          sn[i >> 3][n] = x0;
          sn[i >> 3][n + 1] = x1;
        }
        m = fmaxf(m, x0);
        m = fmaxf(m, x1);
      }
    }
    mx = m;
  };
  // P.V of a wave's last tile (V stage vstage), with no next tile's maxima
  auto pv = [&](int vstage) __attribute__((always_inline)) {
    bf16x8 va[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = v_operand(vstage, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 4 < 16) va[i + 4] = v_operand(vstage, i + 4);
      const int kb = i >> 3, hh = (i >> 2) & 1, db = i & 3;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pf[kb][hh], acc[db], 0, 0, 0);
    }
  };

  // a wave whose 32 rows all lie past Sq (the ragged last q-tile) skips the products
  const bool idle = __builtin_amdgcn_readfirstlane(qt * BM + wave * 32) >= Sq;
  // CAUSAL: the last key tile this wave's rows see (its last valid row's limit; -1: none)
  int wave_last_tile = 0;
  if constexpr (CAUSAL) {
    const int64_t r_w = (int64_t)qt * BM + wave * 32 + 31 < Sq ? (int64_t)qt * BM + wave * 32 + 31 : (int64_t)Sq - 1;
    const int64_t lim_w = r_w + causal_off < (int64_t)Sk - 1 ? r_w + causal_off : (int64_t)Sk - 1;
    wave_last_tile = __builtin_amdgcn_readfirstlane(lim_w < 0 ? -1 : (int)(lim_w / BN));
  }
  // ---- main loop: four LDS stages, tiles loaded three ahead, one barrier per tile ----
  // Tile t lives in stage t % 4.  Iteration t turns the logits of tile t
  // (S[t%2]) into weights while the matrix core computes the logits of tile
  // t+1 (S[(t+1)%2]), then accumulates P.V of tile t while the VALU reduces
  // the row maxima of tile t+1: each wave keeps its matrix core and its VALU
  // busy at the same time.  Before the barrier of iteration t a wave waits
  // for its own loads of tile t+1 (loads complete in order, so those of tile
  // t+2 may remain in flight); the barrier makes every wave's loads visible
  // and frees stage (t+3) % 4, last read in iteration t-1, for the loads of
  // tile t+3.
  auto body = [&](auto st_c, auto masked_c, int t) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value, P = ST & 1;
    if (idle) {
      // no valid row in this wave: only its share of the tile loads and the barrier
      __builtin_amdgcn_s_waitcnt(0x0F74);
      __syncthreads();
      i32x4 rk, rv;
      tile_rsrc(t + 3, rk, rv);
      uint32_t lw = lds_wave;
      asm volatile("" : "+s"(lw));
      dma_k(rk, lw, (ST + 3) % NSTAGE, 0);
      dma_k(rk, lw, (ST + 3) % NSTAGE, 1);
      dma_v(rv, lw, (ST + 3) % NSTAGE, 0);
      dma_v(rv, lw, (ST + 3) % NSTAGE, 1);
      return;
    }
    rescale();
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): only the loads of tile t+2 may still be in flight
    __syncthreads();
    // loads of tile t+3, issued between MFMAs so that a full memory queue
    // stalls this wave while its matrix work is under way
    i32x4 rk, rv;
    tile_rsrc(t + 3, rk, rv);
    uint32_t lw = lds_wave;
    asm volatile("" : "+s"(lw));
    qk_weights(S[1 - P], S[P], k_st[(ST + 1) % NSTAGE],
               [&](int u) __attribute__((always_inline)) { dma_k(rk, lw, (ST + 3) % NSTAGE, u); });
    pv_rowmax(masked_c, ST, S[1 - P], t_begin + t + 1,
              [&](int u) __attribute__((always_inline)) { dma_v(rv, lw, (ST + 3) % NSTAGE, u); });
  };
  // A wave's last iteration with products (tile t in stage ST): its weights and
  // P.V only, since no next tile of this wave needs logits.  SYNC: other waves
  // still have tiles after this one, so the iteration keeps the barrier and
  // this wave's share of the loads; the item's last iteration has neither
  // (the V tile it reads was made visible by the previous barrier).
  auto last_body = [&](auto st_c, bool sync, int t) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value, P = ST & 1;
    if (sync) {
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
      __syncthreads();
      i32x4 rk, rv;
      tile_rsrc(t + 3, rk, rv);
      uint32_t lw = lds_wave;
      asm volatile("" : "+s"(lw));
      dma_k(rk, lw, (ST + 3) % NSTAGE, 0);
      dma_k(rk, lw, (ST + 3) % NSTAGE, 1);
      dma_v(rv, lw, (ST + 3) % NSTAGE, 0);
      dma_v(rv, lw, (ST + 3) % NSTAGE, 1);
    }
    if (idle) return;
    rescale();
    weights(S[P]);
    pv(ST);
  };
  auto last = [&](bool sync, int t) __attribute__((always_inline)) {
    switch (t & 3) {
      case 0: last_body(std::integral_constant<int, 0>{}, sync, t); break;
      case 1: last_body(std::integral_constant<int, 1>{}, sync, t); break;
      case 2: last_body(std::integral_constant<int, 2>{}, sync, t); break;
      default: last_body(std::integral_constant<int, 3>{}, sync, t); break;
    }
  };
  using Plain = std::false_type;
  using Masked = std::true_type;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  // prologue: tiles 0..2 of the visiting order in flight, logits and row
  // maxima of the first (masked when it is the ragged one)
  issue_loads(0, 0);
  issue_loads(1, 1);
  issue_loads(2, 2);
  __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): tile 0 has landed
  __syncthreads();
  qk(S[0], k_st[0]);
  if (CAUSAL) {
    if (t_begin >= diag0) mask_causal(S[0], t_begin);
  } else if (ragged && (!SPLIT || t_begin == 0)) {
    mask_tail(S[0], n_tiles_all - 1);
  }
  rowmax(S[0]);

  if constexpr (CAUSAL) {
    // Iterations compute the logits of the next tile, except a wave's last
    // iteration with products: no tile after it is visible to its rows.
    // Iteration t masks the logits of tile t+1.  The first n_plain
    // iterations (whole rounds of the four stages, their next tiles all
    // before diag0) need no mask; the rest mask whatever tile comes next (a
    // mask on a tile every row sees whole changes nothing).
    const int n_plain = diag0 > t_begin ? min((diag0 - t_begin - 1) & ~3, n_tiles & ~3) : 0;
    int t = 0;
    while (t < n_plain) {
      body(S0{}, Plain{}, t);
      body(S1{}, Plain{}, t + 1);
      body(S2{}, Plain{}, t + 2);
      body(S3{}, Plain{}, t + 3);
      t += 4;
    }
    // Past the last tile its own rows see, a wave's weights are exact zeros
    // and its row maxima -Inf: it leaves the products there and only issues
    // its share of the remaining tile loads, meeting the barrier each tile.
    const int n_w = wave_last_tile - t_begin + 1 < n_tiles ? wave_last_tile - t_begin + 1 : n_tiles;
    while (t < n_w - 1) {
      body(S0{}, Masked{}, t);
      if (++t == n_w - 1) break;
      body(S1{}, Masked{}, t);
      if (++t == n_w - 1) break;
      body(S2{}, Masked{}, t);
      if (++t == n_w - 1) break;
      body(S3{}, Masked{}, t);
      ++t;
    }
    if (t < n_w) {
      last(t + 1 < n_tiles, t);
      ++t;
    }
    for (; t < n_tiles - 1; ++t) {
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
      __syncthreads();
      i32x4 rk, rv;
      tile_rsrc(t + 3, rk, rv);
      const int st = (t + 3) % NSTAGE;
      uint32_t lw = lds_wave;
      asm volatile("" : "+s"(lw));
      dma_k(rk, lw, st, 0);
      dma_k(rk, lw, st, 1);
      dma_v(rv, lw, st, 0);
      dma_v(rv, lw, st, 1);
    }
  } else {
    // Without a mask every iteration runs whole: the last one also computes
    // the logits of a tile that does not exist, and never uses them (peeling
    // that iteration here, in two forms, measured 0.5-1.0% slower, on long
    // items too: it changes how this compiler lays out the loop).  Written as
    // an exit test after each body: a test before the first one makes this
    // compiler spill the pipeline's registers.
    for (int t = 0;;) {
      body(S0{}, Plain{}, t);
      if (++t == n_tiles) break;
      body(S1{}, Plain{}, t);
      if (++t == n_tiles) break;
      body(S2{}, Plain{}, t);
      if (++t == n_tiles) break;
      body(S3{}, Plain{}, t);
      if (++t == n_tiles) break;
    }
  }

  // ---- epilogue ----
  const float l_tot = wave_half_sum(l_run);
  if (SPLIT && slot >= 0) {
    // partial result of a key range: unnormalised rows, m and l
    const int row = wave * 32 + l32;
    float* prow = sp.part + ((int64_t)slot * BM + row) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4*)(prow + 32 * db + 8 * r) =
            f32x4{acc[db][4 * r], acc[db][4 * r + 1], acc[db][4 * r + 2], acc[db][4 * r + 3]};
    if (grp == 0) *(f32x2*)(sp.ml + ((int64_t)slot * BM + row) * 2) = f32x2{m_run, l_tot};
    return;
  }
  // the row's log-sum-exp: the logits of this kernel are t = s log2(e)/sqrt(128),
  // sum_j 2^t_j = 2^m l, so ln(sum_j exp(s_j / sqrt(128))) = ln(2) (m + log2 l)
  // (l = 0: -Inf; l NaN: NaN)
  if (lse && grp == 0 && qrow < Sq) lse[lse_row0 + qrow] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
  if constexpr (MODE == kPartial) {
    // one key shard's rows in fp32, normalised by the shard's own sum (rows
    // that see no key of the shard: 0, with an lse of -Inf)
    const float inv_p = l_tot == 0.0f ? 0.0f : 1.0f / l_tot;
    if (qrow < Sq) {
      float* dst = (float*)O + q_base + h * g.q_head + (int64_t)qrow * g.q_row + 4 * grp;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(f32x4*)(dst + 32 * db + 8 * r) = f32x4{acc[db][4 * r] * inv_p, acc[db][4 * r + 1] * inv_p,
                                                   acc[db][4 * r + 2] * inv_p, acc[db][4 * r + 3] * inv_p};
    }
    return;
  }
  // normalise, round, store this lane's query row
  const float inv_l = 1.0f / l_tot;
  if (qrow < Sq) {
    uint16_t* dst = Oh + (int64_t)qrow * g.q_row + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t lo = round_to_bf16<MODE>(acc[db][4 * r + 0] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 1] * inv_l) << 16);
        uint32_t hi = round_to_bf16<MODE>(acc[db][4 * r + 2] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 3] * inv_l) << 16);
        *(u32x2*)(dst + 32 * db + 8 * r) = u32x2{lo, hi};
      }
  }
}

// Work decomposition.  Whole items: workgroups are dispatched round-robin
// over the 8 XCDs; they are renumbered so that XCD x receives a contiguous
// range of logical work items (a head's q-tiles share one XCD's L2).  Split
// items follow in id order.
// PAIRS (causal mask, fixed-length batches, whole items only): each
// workgroup runs two work items of one head one after the other, q-tiles
// n-1-j and j, so every workgroup sees about the same number of key tiles
// and there are half as many workgroups to start and finish (the hardware
// dispatcher's balancing works on the workgroups as before).  An odd q-tile
// count leaves the middle q-tile of a head alone.  Pairs are numbered over
// the heads (sp.n_whole = their count) and renumbered per XCD like items.
template <int MODE, bool SPLIT, bool CAUSAL, bool VARLEN, bool PAIRS>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, int H, int Sq_all, int Sk_all, int n_qtiles, Geometry g, Split sp, Varlen vl,
    int causal_br, int64_t causal_off_fixed, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * NSTAGE * TILE_BYTES];
  const int id = blockIdx.x;
  const int n_tiles_all = (Sk_all + BN - 1) / BN;
  if constexpr (PAIRS) {
    const int xcd = id & 7, local = id >> 3;
    const int per = sp.n_whole >> 3, rem = sp.n_whole & 7;
    const int pair = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int per_head = (n_qtiles + 1) >> 1;
    const int head = pair / per_head, j = pair % per_head;
    // work items (see attn_item: under a causal mask item w is q-tile n-1-(w % n))
    const int wa = head * n_qtiles + j, wb = head * n_qtiles + n_qtiles - 1 - j;
    const int n_items = n_qtiles - 1 - j != j ? 2 : 1;
    attn_item<MODE, SPLIT, CAUSAL, VARLEN>(Q, K, V, O, H, Sq_all, Sk_all, n_qtiles, g, sp, vl, causal_br,
                                           causal_off_fixed, lse, lds, wa, 0, n_tiles_all, -1);
    if (n_items == 2) {
      // the first item's waves are done with the LDS stages the second one fills
      __syncthreads();
      attn_item<MODE, SPLIT, CAUSAL, VARLEN>(Q, K, V, O, H, Sq_all, Sk_all, n_qtiles, g, sp, vl, causal_br,
                                             causal_off_fixed, lse, lds, wb, 0, n_tiles_all, -1);
    }
  } else {
    int work, t_begin = 0, t_end = n_tiles_all, slot = -1;
    if (!SPLIT || id < sp.n_whole) {
      const int xcd = id & 7, local = id >> 3;
      const int per = sp.n_whole >> 3, rem = sp.n_whole & 7;
      work = xcd * per + (xcd < rem ? xcd : rem) + local;
    } else {
      slot = id - sp.n_whole;
      work = split_item_work(sp, slot / sp.splits, n_qtiles);
      t_begin = (slot % sp.splits) * sp.tiles_per_split;
      t_end = t_begin + sp.tiles_per_split < t_end ? t_begin + sp.tiles_per_split : t_end;
    }
    attn_item<MODE, SPLIT, CAUSAL, VARLEN>(Q, K, V, O, H, Sq_all, Sk_all, n_qtiles, g, sp, vl, causal_br,
                                           causal_off_fixed, lse, lds, work, t_begin, t_end, slot);
  }
}

// Combines the key-range partials of the split work items: per query row,
// M = max_s m_s, w_s = 2^(m_s - M), O = (sum_s w_s o_s) * (1 / sum_s w_s l_s),
// summed in split order, then the one rounding to bf16.  One thread per
// (item, row, 4 dims).  A split whose logits were all -Inf has m_s = -FLT_MAX
// and contributes nothing; a row with no finite logit at all gives 0 * Inf =
// NaN, as in the whole-row kernel.
// reverse_qt: the items of each head are in decreasing q-tile order (the
// causal kernels' order).  With lse, thread 0 of each row also stores the
// row's log-sum-exp, ln(2) (M + log2 L) with L the merged row sum.
template <int MODE>
__global__ __launch_bounds__(256) void attn_merge_kernel(uint16_t* __restrict__ O, int H, int Sq, int n_qtiles,
                                                         Geometry g, Split sp, int n_split_items, int reverse_qt,
                                                         float* __restrict__ lse) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_split_items * BM * (D / 4)) return;
  const int c4 = (int)(gid % (D / 4));
  const int row = (int)((gid / (D / 4)) % BM);
  const int item = (int)(gid / ((D / 4) * BM));
  const int work = split_item_work(sp, item, n_qtiles);
  const int qt = reverse_qt ? n_qtiles - 1 - work % n_qtiles : work % n_qtiles, bh = work / n_qtiles;
  const int h = bh % H, b = bh / H;
  const int qrow = qt * BM + row;
  if (qrow >= Sq) return;
  const int64_t slot0 = (int64_t)item * sp.splits;
  float mmax = -3.402823466e38f;
  for (int s = 0; s < sp.splits; ++s) mmax = fmaxf(mmax, sp.ml[((slot0 + s) * BM + row) * 2]);
  f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  for (int s = 0; s < sp.splits; ++s) {
    const f32x2 ml = *(const f32x2*)(sp.ml + ((slot0 + s) * BM + row) * 2);
    const float w = __builtin_amdgcn_exp2f(ml[0] - mmax);
    const f32x4 o = *(const f32x4*)(sp.part + ((slot0 + s) * BM + row) * D + 4 * c4);
    num += w * o;
    den += w * ml[1];
  }
  if (lse && c4 == 0) lse[((int64_t)b * H + h) * Sq + qrow] = (mmax + log2f(den)) * 0.6931471805599453f;
  const float inv = 1.0f / den;
  uint16_t* dst = O + b * g.q_batch + h * g.q_head + (int64_t)qrow * g.q_row + 4 * c4;
  const uint32_t lo = round_to_bf16<MODE>(num[0] * inv) | ((uint32_t)round_to_bf16<MODE>(num[1] * inv) << 16);
  const uint32_t hi = round_to_bf16<MODE>(num[2] * inv) | ((uint32_t)round_to_bf16<MODE>(num[3] * inv) << 16);
  *(u32x2*)dst = u32x2{lo, hi};
}

// Combines the key-shard partials of attn_fwd_bf16_partial: per query row,
// M = max_s lse_s, w_s = exp(lse_s - M), O = (sum_s w_s O_s) / (sum_s w_s)
// and lse = M + ln(sum_s w_s), summed in shard order, then the one rounding
// to bf16.  One thread per (row, 4 dims); rows are (b, h, i) in row-major
// order, the shards' rows and O at q's element offsets.  A NaN lse in any
// shard makes the row NaN (lse NaN); when no shard has a key for the row
// (every lse -Inf) the row is NaN, the 0/0 of an empty softmax, and its lse
// -Inf.
template <int MODE>
__global__ __launch_bounds__(256) void attn_merge_shards_kernel(const float* __restrict__ parts,
                                                                const float* __restrict__ lse_parts, int n_parts,
                                                                int64_t part_elems, int64_t rows, int H, int Sq,
                                                                Geometry g, uint16_t* __restrict__ O,
                                                                float* __restrict__ lse) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * (D / 4)) return;
  const int c4 = (int)(gid % (D / 4));
  const int64_t row = gid / (D / 4);
  const int i = (int)(row % Sq);
  const int64_t bh = row / Sq;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const int64_t off = b * g.q_batch + h * g.q_head + (int64_t)i * g.q_row + 4 * c4;
  float mmax = -__builtin_inff();
  bool nan = false;
  for (int s = 0; s < n_parts; ++s) {
    const float x = lse_parts[(int64_t)s * rows + row];
    nan |= x != x;
    mmax = fmaxf(mmax, x);
  }
  f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f, lse_row;
  if (nan || mmax == -__builtin_inff()) {
    const float qnan = __builtin_nanf("");
    num = f32x4{qnan, qnan, qnan, qnan};
    den = 1.0f;
    lse_row = nan ? qnan : -__builtin_inff();
  } else {
    for (int s = 0; s < n_parts; ++s) {
      const float w = __builtin_amdgcn_exp2f((lse_parts[(int64_t)s * rows + row] - mmax) * 1.4426950408889634f);
      const f32x4 o = *(const f32x4*)(parts + (int64_t)s * part_elems + off);
      num += w * o;
      den += w;
    }
    lse_row = mmax + log2f(den) * 0.6931471805599453f;
  }
  if (lse && c4 == 0) lse[row] = lse_row;
  const float inv = 1.0f / den;
  const uint32_t lo = round_to_bf16<MODE>(num[0] * inv) | ((uint32_t)round_to_bf16<MODE>(num[1] * inv) << 16);
  const uint32_t hi = round_to_bf16<MODE>(num[2] * inv) | ((uint32_t)round_to_bf16<MODE>(num[3] * inv) << 16);
  *(u32x2*)(O + off) = u32x2{lo, hi};
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cu_count[kMaxDevices];    // 0 unknown

// The current device must be gfx950 (its CU count is cached), and a stream the
// caller passes must belong to it: the split plans use this device's CU count
// and the static scratch is this device's.  A stream whose device cannot be
// queried is taken as it is.
int check_device(int* n_cu, void* stream = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) == hipSuccess && sdev != dev) return ATTN_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 2) return ATTN_ERR_DEVICE;
    if (st == 1) {
      *n_cu = g_cu_count[dev].load(std::memory_order_relaxed);
      return ATTN_OK;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.multiProcessorCount > 0;
  *n_cu = prop.multiProcessorCount;
  if (dev < kMaxDevices) {
    g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  }
  return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

// Static scratch of attn_fwd_bf16_gqa_noalloc: the split path's partial rows
// and (m, l) pairs, for callers that cannot allocate (graph capture, tight
// serving loops).  Sized for the largest plan on a 256-CU device: 2 x 256
// partial blocks of BM rows x (D + 2) floats (65 MiB).  Every GPU the library
// runs on holds its own copy until the process ends; host code reaches it
// only through the address hipGetSymbolAddress gives for the current device
// (the array's name on the host is a stand-in, not a device address).
constexpr int64_t kScratchBytes = int64_t(2) * 256 * BM * (D + 2) * (int64_t)sizeof(float);
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device (looked up once per
// device, with that device current), or nullptr when the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    g_scratch[dev].store(addr, std::memory_order_release);
    p = addr;
  }
  return p;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Launch kern on stream s and return that launch's own status: hipGetLastError
// would also report (and clear) an error that an earlier call of the caller
// left behind.  The arguments are converted to the kernel's parameter types
// and passed by address, one pointer per parameter.
template <typename K, typename T, size_t... I>
hipError_t launch_args(K kern, dim3 grid, dim3 block, hipStream_t s, T& args, std::index_sequence<I...>) {
  void* ptrs[] = {(void*)&std::get<I>(args)...};
  return hipLaunchKernel((const void*)kern, grid, block, ptrs, 0, s);
}
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<P...> args(std::forward<A>(a)...);
  return launch_args(kern, grid, block, s, args, std::index_sequence_for<P...>{});
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Split plan for n_work items of n_tiles key tiles on n_cu compute units
// (one workgroup per CU at a time).  When the items do not fill the last
// round of CUs, the items of that round run as several key ranges each, so
// the round holds as many workgroups as there are CUs; a range holds at
// least kMinSplitTiles tiles.
constexpr int kMinSplitTiles = 4;
struct Plan {
  int64_t n_whole, n_split_items, splits, tiles_per_split;
  int64_t qt_major = 0;  // Split::qt_major
};
Plan make_plan(int64_t n_work, int64_t n_tiles, int64_t n_cu) {
  Plan p{n_work, 0, 1, n_tiles};
  if (n_cu < 1 || n_work % n_cu == 0) return p;
  const int64_t n_tail = n_work % n_cu;
  int64_t splits = n_cu / n_tail;
  if (splits > n_tiles / kMinSplitTiles) splits = n_tiles / kMinSplitTiles;
  if (splits < 2) return p;
  const int64_t tps = (n_tiles + splits - 1) / splits;
  splits = (n_tiles + tps - 1) / tps;  // every range non-empty
  if (splits < 2) return p;
  p.n_whole = n_work - n_tail;
  p.n_split_items = n_tail;
  p.splits = splits;
  p.tiles_per_split = tps;
  return p;
}
// Key tiles the q-tile qt visits under a causal mask (row i sees keys
// j <= i + off, off = 0 or Sk - Sq): up to its last row's limit, and one
// (fully masked) tile when no row sees a key.
int64_t causal_tiles(int64_t qt, int64_t Sq, int64_t Sk, int mask) {
  const int64_t off = mask == ATTN_MASK_CAUSAL_BOTTOM_RIGHT ? Sk - Sq : 0;
  const int64_t r_last = (qt * BM + BM < Sq ? qt * BM + BM : Sq) - 1;
  const int64_t hi = r_last + off < Sk - 1 ? r_last + off : Sk - 1;
  return hi < 0 ? 1 : hi / BN + 1;
}
// Split plan under a mask.  The items of a causal launch differ in length.
// When they are nearly equal (the lightest q-tile visits at least 3/4 of the
// tiles of the heaviest, as when Sq is small against Sk with the bottom-right
// diagonal) only the partly idle last round is split, as without a mask.
// When they are not, several rounds of items keep the CUs busy to the end in
// the longest-first order, but one round or less does not: the longest item
// alone sets the time, about twice the mean load.  Then every item is cut
// into `splits` ranges of its own visible tiles, up to twice as many
// workgroups as CUs (at most 8 ranges an item, each at least kMinSplitTiles
// tiles of the longest item).
Plan make_plan_masked(int64_t n_work, int64_t n_qtiles, int64_t Sq, int64_t Sk, int mask, int64_t n_cu) {
  if (mask == ATTN_MASK_NONE) return make_plan(n_work, (Sk + BN - 1) / BN, n_cu);
  const int64_t n_max = causal_tiles(n_qtiles - 1, Sq, Sk, mask), n_min = causal_tiles(0, Sq, Sk, mask);
  if (4 * n_min >= 3 * n_max) return make_plan(n_work, n_max, n_cu);
  const Plan whole{n_work, 0, 1, n_max};
  if (n_cu < 1 || n_work > n_cu) return whole;
  int64_t splits = 2 * n_cu / n_work;
  if (splits > 8) splits = 8;
  if (splits > n_max / kMinSplitTiles) splits = n_max / kMinSplitTiles;
  if (splits < 2) return whole;
  // all items split, dispatched longest q-tile first across the heads (the
  // ranges of one q-tile rank are nearly equal): in head order the longest
  // items of the last heads would start last
  return Plan{0, n_work, splits, (n_max + splits - 1) / splits, n_work / n_qtiles};
}
int64_t plan_workspace_bytes(const Plan& p) {
  return p.n_split_items * p.splits * BM * (D + 2) * (int64_t)sizeof(float);
}

struct Problem {
  int64_t bytes_q, bytes_k, n_work, n_qtiles, n_tiles;
};
// argument checks shared by the entry points (no HIP calls)
int check_args(const void* q, const void* k, const void* v, const void* o, int64_t B, int64_t H, int64_t H_kv,
               int64_t Sq, int64_t Sk, int layout, int round_mode, Problem* pb) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || H_kv < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SIZE;
  if (H % H_kv != 0) return ATTN_ERR_HEADS;
  int64_t bh, bhk, nq, nk;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, Sq, &nq) || !mul_ok(nq, 2 * D, &pb->bytes_q) || !mul_ok(B, H_kv, &bhk) ||
      !mul_ok(bhk, Sk, &nk) || !mul_ok(nk, 2 * D, &pb->bytes_k))
    return ATTN_ERR_SIZE;
  pb->n_qtiles = (Sq + BM - 1) / BM;
  pb->n_tiles = (Sk + BN - 1) / BN;
  if (!mul_ok(bh, pb->n_qtiles, &pb->n_work) || pb->n_work > INT32_MAX - 65536 || Sq > INT32_MAX ||
      Sk > INT32_MAX || H > kMaxHeads)
    return ATTN_ERR_SIZE;
  if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
  if (round_mode != ATTN_ROUND_RTNE && round_mode != ATTN_ROUND_RTNA && round_mode != ATTN_ROUND_RTZ)
    return ATTN_ERR_ROUND;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if (overlaps(o, pb->bytes_q, q, pb->bytes_q) || overlaps(o, pb->bytes_q, k, pb->bytes_k) ||
      overlaps(o, pb->bytes_q, v, pb->bytes_k))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

Geometry make_geometry(int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout) {
  Geometry g;
  if (layout == ATTN_LAYOUT_BSHD) {
    g.q_row = H * D;
    g.k_row = H_kv * D;
    g.q_head = D;
    g.k_head = D;
    g.q_batch = Sq * H * D;
    g.k_batch = Sk * H_kv * D;
  } else {
    g.q_row = D;
    g.k_row = D;
    g.q_head = Sq * D;
    g.k_head = Sk * D;
    g.q_batch = H * Sq * D;
    g.k_batch = H_kv * Sk * D;
  }
  g.kv_group = H / H_kv;
  return g;
}

template <int MODE>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int H, int Sq, int Sk,
                  int n_qtiles, const Geometry& g, const Split& sp, const Varlen* vl, int64_t n_wg,
                  int n_split_items, int mask, float* lse, bool pairs, hipStream_t s) {
  const int br = mask == ATTN_MASK_CAUSAL_BOTTOM_RIGHT;
  const int64_t off = br ? (int64_t)Sk - Sq : 0;  // fixed-length calls: row i sees keys j <= i + off
  const Varlen none{nullptr, nullptr, 0, 0, 0};
  const dim3 grid((unsigned)n_wg), block(NTHREADS);
  if (pairs) {
    // two work items per workgroup (fixed-length, no split): n_wg counts the pairs
    Split spp = sp;
    spp.n_whole = (int)n_wg;
    return launch_kernel(attn_fwd_kernel<MODE, false, true, false, true>, grid, block, s, q, k, v, o, H, Sq, Sk,
                         n_qtiles, g, spp, none, 0, off, lse);
  }
  hipError_t e;
  if (n_split_items > 0 && mask != ATTN_MASK_NONE)
    e = launch_kernel(attn_fwd_kernel<MODE, true, true, false, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, none, 0, off, lse);
  else if (n_split_items > 0)
    e = launch_kernel(attn_fwd_kernel<MODE, true, false, false, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, none, 0, (int64_t)0, lse);
  else if (vl && mask != ATTN_MASK_NONE)
    e = launch_kernel(attn_fwd_kernel<MODE, false, true, true, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, *vl, br, (int64_t)0, lse);
  else if (vl)
    e = launch_kernel(attn_fwd_kernel<MODE, false, false, true, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, *vl, 0, (int64_t)0, lse);
  else if (mask != ATTN_MASK_NONE)
    e = launch_kernel(attn_fwd_kernel<MODE, false, true, false, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, none, 0, off, lse);
  else
    e = launch_kernel(attn_fwd_kernel<MODE, false, false, false, false>, grid, block, s, q, k, v, o, H, Sq, Sk,
                      n_qtiles, g, sp, none, 0, (int64_t)0, lse);
  if (e == hipSuccess && n_split_items > 0) {
    const int64_t threads = (int64_t)n_split_items * BM * (D / 4);
    e = launch_kernel(attn_merge_kernel<MODE>, dim3((unsigned)((threads + 255) / 256)), dim3(256), s, o, H, Sq,
                      n_qtiles, g, sp, n_split_items, mask != ATTN_MASK_NONE ? 1 : 0, lse);
  }
  return e;
}

int run(const void* q, const void* k, const void* v, void* o, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk,
        int layout, int round_mode, int mask, const Problem& pb, const Plan& plan, void* workspace, void* stream,
        int n_cu, const Varlen* vl = nullptr, float* lse = nullptr) {
  const Geometry g = make_geometry(H, H_kv, Sq, Sk, layout);
  Split sp{(int)plan.n_whole, (int)plan.splits, (int)plan.tiles_per_split, nullptr, nullptr, (int)plan.qt_major};
  if (plan.n_split_items > 0) {
    sp.part = (float*)workspace;
    sp.ml = sp.part + plan.n_split_items * plan.splits * BM * D;
  }
  int64_t n_wg = plan.n_whole + plan.n_split_items * plan.splits;
  // causal whole fixed-length items in at least two rounds of compute units: two per workgroup
  // (without a mask the items are equal already, and one per workgroup measured faster)
  const bool pairs =
      mask != ATTN_MASK_NONE && !vl && plan.n_split_items == 0 && n_cu > 0 && pb.n_work >= 2 * (int64_t)n_cu;
  if (pairs) n_wg = pb.n_work / pb.n_qtiles * ((pb.n_qtiles + 1) / 2);
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  uint16_t* oo = (uint16_t*)o;
  hipStream_t s = (hipStream_t)stream;
  const int nsi = (int)plan.n_split_items;
  hipError_t e;
  switch (round_mode) {
    case ATTN_ROUND_RTNE:
      e = launch<ATTN_ROUND_RTNE>(qq, kk, vv, oo, (int)H, (int)Sq, (int)Sk, (int)pb.n_qtiles, g, sp, vl, n_wg, nsi,
                                  mask, lse, pairs, s);
      break;
    case ATTN_ROUND_RTNA:
      e = launch<ATTN_ROUND_RTNA>(qq, kk, vv, oo, (int)H, (int)Sq, (int)Sk, (int)pb.n_qtiles, g, sp, vl, n_wg, nsi,
                                  mask, lse, pairs, s);
      break;
    default:
      e = launch<ATTN_ROUND_RTZ>(qq, kk, vv, oo, (int)H, (int)Sq, (int)Sk, (int)pb.n_qtiles, g, sp, vl, n_wg, nsi,
                                 mask, lse, pairs, s);
      break;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                             int64_t Sq, int64_t Sk, int layout, int round_mode, void* stream) {
  Problem pb;
  const int st = check_args(q, k, v, o, B, H, H, Sq, Sk, layout, round_mode, &pb);
  if (st != ATTN_OK) return st;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  const Plan whole{pb.n_work, 0, 1, pb.n_tiles};
  return run(q, k, v, o, H, H, Sq, Sk, layout, round_mode, ATTN_MASK_NONE, pb, whole, nullptr, stream, n_cu);
}

extern "C" int attn_fwd_bf16_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                 int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int round_mode,
                                 int mask, void* stream) {
  Problem pb;
  const int st = check_args(q, k, v, o, B, H, H_kv, Sq, Sk, layout, round_mode, &pb);
  if (st != ATTN_OK) return st;
  if (lse) {
    // [B, H, Sq] fp32; B*H*Sq*256 is the (checked) size of q, so this fits
    const int64_t lse_bytes = pb.bytes_q / 64;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    if (overlaps(lse, lse_bytes, q, pb.bytes_q) || overlaps(lse, lse_bytes, k, pb.bytes_k) ||
        overlaps(lse, lse_bytes, v, pb.bytes_k) || overlaps(lse, lse_bytes, o, pb.bytes_q))
      return ATTN_ERR_ALIAS;
  }
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  const Plan whole{pb.n_work, 0, 1, pb.n_tiles};
  return run(q, k, v, o, H, H_kv, Sq, Sk, layout, round_mode, mask, pb, whole, nullptr, stream, n_cu, nullptr, lse);
}

extern "C" int attn_fwd_bf16_masked(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                                    int64_t Sq, int64_t Sk, int layout, int round_mode, int mask, void* stream) {
  return attn_fwd_bf16_gqa(q, k, v, o, nullptr, B, H, H, Sq, Sk, layout, round_mode, mask, stream);
}

extern "C" int attn_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B, int64_t H,
                                    int64_t H_kv, int64_t total_q, int64_t total_k, int64_t max_seqlen_q,
                                    int round_mode, int mask, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || H_kv < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1) return ATTN_ERR_SIZE;
  if (H % H_kv != 0) return ATTN_ERR_HEADS;
  Problem pb;
  int64_t rows_q, rows_k;
  if (B > INT32_MAX - 1 || total_q > INT32_MAX || total_k > INT32_MAX || max_seqlen_q > INT32_MAX ||
      H > kMaxHeads || !mul_ok(total_q, H, &rows_q) || !mul_ok(rows_q, 2 * D, &pb.bytes_q) ||
      !mul_ok(total_k, H_kv, &rows_k) || !mul_ok(rows_k, 2 * D, &pb.bytes_k))
    return ATTN_ERR_SIZE;
  pb.n_qtiles = (max_seqlen_q + BM - 1) / BM;
  pb.n_tiles = 1;
  int64_t bh;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, pb.n_qtiles, &pb.n_work) || pb.n_work > INT32_MAX - 65536)
    return ATTN_ERR_SIZE;
  if (round_mode != ATTN_ROUND_RTNE && round_mode != ATTN_ROUND_RTNA && round_mode != ATTN_ROUND_RTZ)
    return ATTN_ERR_ROUND;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) ||
      (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3))
    return ATTN_ERR_ALIGN;
  const int64_t cu_bytes = (B + 1) * 4;
  if (overlaps(o, pb.bytes_q, q, pb.bytes_q) || overlaps(o, pb.bytes_q, k, pb.bytes_k) ||
      overlaps(o, pb.bytes_q, v, pb.bytes_k) || overlaps(o, pb.bytes_q, cu_seqlens_q, cu_bytes) ||
      overlaps(o, pb.bytes_q, cu_seqlens_k, cu_bytes))
    return ATTN_ERR_ALIAS;
  if (lse) {
    // [H, total_q] fp32
    const int64_t lse_bytes = pb.bytes_q / 64;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    if (overlaps(lse, lse_bytes, q, pb.bytes_q) || overlaps(lse, lse_bytes, k, pb.bytes_k) ||
        overlaps(lse, lse_bytes, v, pb.bytes_k) || overlaps(lse, lse_bytes, o, pb.bytes_q) ||
        overlaps(lse, lse_bytes, cu_seqlens_q, cu_bytes) || overlaps(lse, lse_bytes, cu_seqlens_k, cu_bytes))
      return ATTN_ERR_ALIAS;
  }
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  // grid: 8 XCDs x ceil(groups / 8) groups each x the items of a group
  const int64_t n_groups = B * H_kv, per_group = (H / H_kv) * pb.n_qtiles;
  int64_t n_wg;
  if (!mul_ok(8 * ((n_groups + 7) / 8), per_group, &n_wg) || n_wg > INT32_MAX - 65536) return ATTN_ERR_SIZE;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  const Varlen vl{cu_seqlens_q, cu_seqlens_k, (int)total_q, (int)total_k, (int)n_groups};
  pb.n_work = n_wg;
  const Plan whole{pb.n_work, 0, 1, pb.n_tiles};
  return run(q, k, v, o, H, H_kv, max_seqlen_q, 1, ATTN_LAYOUT_BSHD, round_mode, mask, pb, whole, nullptr, stream,
             n_cu, &vl, lse);
}

extern "C" int attn_fwd_bf16_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                                     int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t key_offset,
                                     int64_t Sk_total, int layout, int mask, void* stream) {
  Problem pb;
  const int st = check_args(q, k, v, o_part, B, H, H_kv, Sq, Sk, layout, ATTN_ROUND_RTNE, &pb);
  if (st != ATTN_OK) return st;
  if (!lse_part) return ATTN_ERR_NULL;
  if (key_offset < 0 || Sk_total > INT32_MAX || key_offset > Sk_total - Sk) return ATTN_ERR_SIZE;
  if ((uintptr_t)lse_part & 3) return ATTN_ERR_ALIGN;
  // fp32 rows: twice q's bytes; the lse: a 64th of q's bytes
  const int64_t o_bytes = 2 * pb.bytes_q, lse_bytes = pb.bytes_q / 64;
  if (overlaps(o_part, o_bytes, q, pb.bytes_q) || overlaps(o_part, o_bytes, k, pb.bytes_k) ||
      overlaps(o_part, o_bytes, v, pb.bytes_k) || overlaps(lse_part, lse_bytes, q, pb.bytes_q) ||
      overlaps(lse_part, lse_bytes, k, pb.bytes_k) || overlaps(lse_part, lse_bytes, v, pb.bytes_k) ||
      overlaps(lse_part, lse_bytes, o_part, o_bytes))
    return ATTN_ERR_ALIAS;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  // row i sees the global keys j <= i + off_global; this shard's key j is
  // global key key_offset + j
  const int64_t off_global = mask == ATTN_MASK_CAUSAL_BOTTOM_RIGHT ? Sk_total - Sq : 0;
  const int64_t off = off_global - key_offset;
  const Geometry g = make_geometry(H, H_kv, Sq, Sk, layout);
  const Split sp{(int)pb.n_work, 1, (int)pb.n_tiles, nullptr, nullptr, 0};
  const Varlen none{nullptr, nullptr, 0, 0, 0};
  const dim3 grid((unsigned)pb.n_work), block(NTHREADS);
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  uint16_t* oo = (uint16_t*)o_part;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e =
      mask == ATTN_MASK_NONE
          ? launch_kernel(attn_fwd_kernel<kPartial, false, false, false, false>, grid, block, s, qq, kk, vv, oo,
                          (int)H, (int)Sq, (int)Sk, (int)pb.n_qtiles, g, sp, none, 0, (int64_t)0, lse_part)
          : launch_kernel(attn_fwd_kernel<kPartial, false, true, false, false>, grid, block, s, qq, kk, vv, oo,
                          (int)H, (int)Sq, (int)Sk, (int)pb.n_qtiles, g, sp, none, 0, off, lse_part);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_bf16_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o,
                                   float* lse, int64_t B, int64_t H, int64_t Sq, int layout, int round_mode,
                                   void* stream) {
  if (!o_parts || !lse_parts || !o) return ATTN_ERR_NULL;
  int64_t bh, rows, part_bytes, all_parts, lse_all, o_bytes;
  if (n_parts < 1 || B < 1 || H < 1 || Sq < 1 || n_parts > INT32_MAX || Sq > INT32_MAX || H > kMaxHeads ||
      !mul_ok(B, H, &bh) || !mul_ok(bh, Sq, &rows) || !mul_ok(rows, 4 * D, &part_bytes) ||
      !mul_ok(part_bytes, n_parts, &all_parts) || !mul_ok(rows * 4, n_parts, &lse_all) ||
      rows > (int64_t(1) << 35))  // the grid of rows * 32 threads in 256-thread blocks fits 32 bits
    return ATTN_ERR_SIZE;
  o_bytes = part_bytes / 2;
  if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
  if (round_mode != ATTN_ROUND_RTNE && round_mode != ATTN_ROUND_RTNA && round_mode != ATTN_ROUND_RTZ)
    return ATTN_ERR_ROUND;
  if ((((uintptr_t)o_parts | (uintptr_t)o) & 15) || (((uintptr_t)lse_parts | (uintptr_t)lse) & 3))
    return ATTN_ERR_ALIGN;
  if (overlaps(o, o_bytes, o_parts, all_parts) || overlaps(o, o_bytes, lse_parts, lse_all) ||
      (lse && (overlaps(lse, rows * 4, o_parts, all_parts) || overlaps(lse, rows * 4, lse_parts, lse_all) ||
               overlaps(lse, rows * 4, o, o_bytes))))
    return ATTN_ERR_ALIAS;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  const Geometry g = make_geometry(H, H, Sq, 1, layout);
  const int64_t threads = rows * (D / 4);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  hipStream_t s = (hipStream_t)stream;
  uint16_t* oo = (uint16_t*)o;
  const int64_t part_elems = rows * D;
  hipError_t e;
  switch (round_mode) {
    case ATTN_ROUND_RTNE:
      e = launch_kernel(attn_merge_shards_kernel<ATTN_ROUND_RTNE>, grid, block, s, o_parts, lse_parts, (int)n_parts,
                        part_elems, rows, (int)H, (int)Sq, g, oo, lse);
      break;
    case ATTN_ROUND_RTNA:
      e = launch_kernel(attn_merge_shards_kernel<ATTN_ROUND_RTNA>, grid, block, s, o_parts, lse_parts, (int)n_parts,
                        part_elems, rows, (int)H, (int)Sq, g, oo, lse);
      break;
    default:
      e = launch_kernel(attn_merge_shards_kernel<ATTN_ROUND_RTZ>, grid, block, s, o_parts, lse_parts, (int)n_parts,
                        part_elems, rows, (int)H, (int)Sq, g, oo, lse);
      break;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_bf16_split_plan(int64_t n_work, int64_t n_tiles, int64_t n_cu, int64_t* out4) {
  if (!out4) return ATTN_ERR_NULL;
  if (n_work < 1 || n_tiles < 1 || n_cu < 1) return ATTN_ERR_SIZE;
  const Plan p = make_plan(n_work, n_tiles, n_cu);
  out4[0] = p.n_whole;
  out4[1] = p.n_split_items;
  out4[2] = p.splits;
  out4[3] = p.tiles_per_split;
  return ATTN_OK;
}

extern "C" int attn_fwd_bf16_split_plan_masked(int64_t n_heads, int64_t Sq, int64_t Sk, int mask, int64_t n_cu,
                                               int64_t* out4) {
  if (!out4) return ATTN_ERR_NULL;
  int64_t n_work;
  if (n_heads < 1 || Sq < 1 || Sk < 1 || n_cu < 1 || Sq > INT32_MAX || Sk > INT32_MAX ||
      !mul_ok(n_heads, (Sq + BM - 1) / BM, &n_work))
    return ATTN_ERR_SIZE;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  const Plan p = make_plan_masked(n_work, (Sq + BM - 1) / BM, Sq, Sk, mask, n_cu);
  out4[0] = p.n_whole;
  out4[1] = p.n_split_items;
  out4[2] = p.splits;
  out4[3] = p.tiles_per_split;
  return ATTN_OK;
}

extern "C" int attn_fwd_bf16_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL;
  *bytes = 0;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SIZE;
  int64_t bh, n_work;
  const int64_t n_qtiles = (Sq + BM - 1) / BM;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, n_qtiles, &n_work) || n_work > INT32_MAX - 65536 || Sk > INT32_MAX)
    return ATTN_ERR_SIZE;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu);
  if (dev_status != ATTN_OK) return dev_status;
  *bytes = plan_workspace_bytes(make_plan(n_work, (Sk + BN - 1) / BN, n_cu));
  return ATTN_OK;
}

extern "C" int attn_fwd_bf16_gqa_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int mask,
                                                int64_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL;
  *bytes = 0;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SIZE;
  int64_t bh, n_work;
  const int64_t n_qtiles = (Sq + BM - 1) / BM;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, n_qtiles, &n_work) || n_work > INT32_MAX - 65536 || Sq > INT32_MAX ||
      Sk > INT32_MAX)
    return ATTN_ERR_SIZE;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu);
  if (dev_status != ATTN_OK) return dev_status;
  *bytes = plan_workspace_bytes(make_plan_masked(n_work, n_qtiles, Sq, Sk, mask, n_cu));
  return ATTN_OK;
}

namespace {
// attn_fwd_bf16_gqa_ws, with the workspace given (noalloc false) or the
// static scratch of the current device (noalloc true)
int gqa_split_call(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int round_mode, int mask, void* workspace,
                   int64_t workspace_bytes, void* stream, bool noalloc) {
  Problem pb;
  const int st = check_args(q, k, v, o, B, H, H_kv, Sq, Sk, layout, round_mode, &pb);
  if (st != ATTN_OK) return st;
  if (lse) {
    const int64_t lse_bytes = pb.bytes_q / 64;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    if (overlaps(lse, lse_bytes, q, pb.bytes_q) || overlaps(lse, lse_bytes, k, pb.bytes_k) ||
        overlaps(lse, lse_bytes, v, pb.bytes_k) || overlaps(lse, lse_bytes, o, pb.bytes_q))
      return ATTN_ERR_ALIAS;
  }
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_MASK;
  if (workspace_bytes < 0) return ATTN_ERR_SIZE;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  const Plan plan = make_plan_masked(pb.n_work, pb.n_qtiles, Sq, Sk, mask, n_cu);
  const int64_t need = plan_workspace_bytes(plan);
  if (need > 0 && noalloc) {
    if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
    workspace = scratch_address();
    if (!workspace) return ATTN_ERR_HIP;
  } else if (need > 0) {
    if (!workspace) return ATTN_ERR_NULL;
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15) return ATTN_ERR_ALIGN;
    if (overlaps(workspace, need, q, pb.bytes_q) || overlaps(workspace, need, k, pb.bytes_k) ||
        overlaps(workspace, need, v, pb.bytes_k) || overlaps(workspace, need, o, pb.bytes_q) ||
        (lse && overlaps(workspace, need, lse, pb.bytes_q / 64)))
      return ATTN_ERR_ALIAS;
  }
  return run(q, k, v, o, H, H_kv, Sq, Sk, layout, round_mode, mask, pb, plan, workspace, stream, n_cu, nullptr,
             lse);
}
}  // namespace

extern "C" int attn_fwd_bf16_gqa_ws(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                    int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout, int round_mode,
                                    int mask, void* workspace, int64_t workspace_bytes, void* stream) {
  return gqa_split_call(q, k, v, o, lse, B, H, H_kv, Sq, Sk, layout, round_mode, mask, workspace, workspace_bytes,
                        stream, false);
}

extern "C" int attn_fwd_bf16_gqa_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                         int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int layout,
                                         int round_mode, int mask, void* stream) {
  return gqa_split_call(q, k, v, o, lse, B, H, H_kv, Sq, Sk, layout, round_mode, mask, nullptr, 0, stream, true);
}

extern "C" int attn_fwd_bf16_ws(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                                int64_t Sq, int64_t Sk, int layout, int round_mode, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  Problem pb;
  const int st = check_args(q, k, v, o, B, H, H, Sq, Sk, layout, round_mode, &pb);
  if (st != ATTN_OK) return st;
  if (workspace_bytes < 0) return ATTN_ERR_SIZE;
  int n_cu = 0;
  const int dev_status = check_device(&n_cu, stream);
  if (dev_status != ATTN_OK) return dev_status;
  Plan plan = make_plan(pb.n_work, pb.n_tiles, n_cu);
  const int64_t need = plan_workspace_bytes(plan);
  if (need > 0) {
    if (!workspace) return ATTN_ERR_NULL;
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15) return ATTN_ERR_ALIGN;
    if (overlaps(workspace, need, q, pb.bytes_q) || overlaps(workspace, need, k, pb.bytes_k) ||
        overlaps(workspace, need, v, pb.bytes_k) || overlaps(workspace, need, o, pb.bytes_q))
      return ATTN_ERR_ALIAS;
  }
  return run(q, k, v, o, H, H, Sq, Sk, layout, round_mode, ATTN_MASK_NONE, pb, plan, workspace, stream, n_cu);
}

extern "C" const char* attn_fwd_bf16_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a tensor or workspace pointer is NULL";
    case ATTN_ERR_SIZE: return "B, H, Sq and Sk must be >= 1 and the problem must fit the index types";
    case ATTN_ERR_LAYOUT: return "layout must be ATTN_LAYOUT_BSHD or ATTN_LAYOUT_BHSD";
    case ATTN_ERR_ROUND: return "round_mode must be ATTN_ROUND_RTNE, ATTN_ROUND_RTNA or ATTN_ROUND_RTZ";
    case ATTN_ERR_ALIGN: return "q, k, v, o and the workspace must be 16-byte aligned";
    case ATTN_ERR_ALIAS: return "o or the workspace overlaps another buffer";
    case ATTN_ERR_DEVICE:
      return "the current HIP device is not gfx950 (MI355X) or cannot be queried, or the stream belongs to another "
             "device";
    case ATTN_ERR_HIP: return "the HIP kernel launch failed";
    case ATTN_ERR_WORKSPACE: return "the workspace is smaller than attn_fwd_bf16_workspace_size reports";
    case ATTN_ERR_MASK: return "mask is not an attn_mask_t value";
    case ATTN_ERR_HEADS: return "the query head count is not a multiple of the K/V head count";
    case ATTN_ERR_SCRATCH: return "the split needs more scratch than the static buffer of attn_fwd_bf16_gqa_noalloc holds";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_bf16_abi_version(void) { return ATTN_FWD_ABI_VERSION; }
