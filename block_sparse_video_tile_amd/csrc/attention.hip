// Block-sparse flash-attention forward for the VSA hot path on gfx950 (CDNA4).
//
// "FastVideo VSA" user guide, intro: exact attention runs only against the
// selected key/value blocks of each query block; "Verify routing and
// fallback": non-causal, equal Q/KV lengths, scale head_size**-0.5, equal
// head counts, no mask.  FastVideo h3-perf-stack commit log, sm_100a tile-64
// route entry: rows of a compacted block map may hold different numbers of
// blocks, including none.
//
// Work decomposition
//   One workgroup per CSR row r = (b*NH + h)*nb + i, i.e. one query block of
//   V = 32*NQ tokens; wave w owns query rows 32w .. 32w+31 (in an 8-wave
//   block cut by the grid edge to 5 or 6 row groups, waves 4..7 instead share
//   the last groups by key halves, and with at most 4 groups waves w and w+4
//   share group w: see the key-half waves below; a 64-token block runs 4
//   waves, two per query group, each group's keys split between them the same
//   way, so that two workgroups of a CU put two waves on every SIMD).  The
//   8-wave blocked kernel runs the alternating pipeline described at
//   pp_pipeline (waves 0..3 and 4..7 take turns on the matrix cores, rings of
//   four K and three V sub-tiles); the others the interleaved step below.
//   Row ids are
//   remapped so that each of the 8 XCDs (workgroups are dispatched to XCDs
//   round-robin) works through a contiguous range of rows, i.e. the same
//   heads, and its L2 serves their shared key/value blocks.  In the balanced
//   launch the same ranges are queues from which the workgroups claim their
//   rows at run time (claim_row), so XCDs that run faster take more rows;
//   for a caller's block map the rows of each queue are first put in claim
//   order (order_rows_kernel: long rows first, then head by head by entry
//   count, so that the workgroups of an XCD stream a head's key blocks in
//   step and share them in L2); for a
//   layer whose heads' key/value blocks outgrow the memory-side cache when
//   the XCDs work on 8 different heads, the queues interleave the heads
//   instead (claim_row_strided).  Launches of at most 256 rows per queue
//   (a few rounds of rows per CU) hand out the last rows of each queue as
//   two halves of their entries, merged by the half that finishes second
//   (the tail split, see TailSplit), so the kernel's last round is made of
//   half rows.
//   The row's key blocks are streamed in 64-key sub-tiles (a block with c
//   valid tokens has ceil(c/64) of them; trailing all-pad sub-tiles are never
//   loaded).  The workgroup first flattens its CSR entries into a list of
//   sub-tile descriptors in LDS, so the main loop carries no CSR walking, no
//   divisions and no global index loads; the descriptor three sub-tiles ahead
//   is read from LDS while the current one is being computed.
//   K (64 x 128) and V^T (128 x 64) sub-tiles are copied HBM/L2 -> LDS
//   directly (global_load_lds_dwordx4, no VGPR staging).  In the interleaved
//   step they are double-buffered, one barrier per sub-tile; with 8 or 6
//   waves (the raster kernel) the copies are issued from
//   inside the MFMA slots (K in the QK^T half, V in the PV half) rather than
//   as one burst; the 4-wave kernels, whose 64-key steps are too short to
//   hide them that way, issue theirs at the top of each step.  K runs one
//   sub-tile ahead of V so that the next sub-tile's QK^T can run on the
//   matrix cores while this sub-tile's softmax runs on the VALU (software
//   pipeline inside each wave).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, or _f16 for fp16 tensors;
// D[m][n] += A[m][k] B[k][n];
// lane l holds A row m = l%32, B column n = l%32, and accumulator register
// j holds row m = 8*(j/4) + 4*(l/32) + j%4 of column n = l%32):
//   S^T = K Q^T :  A = K sub-tile rows (keys) from LDS, B = Q^T fragments
//                  kept in VGPRs for the whole row.  Each lane then holds 32
//                  scores of ONE query (column n), so the softmax max and sum
//                  are in-lane plus one exchange between lanes l and l^32.
//   O^T += V^T P^T: A = V^T rows (d) from LDS, B = P^T taken straight from the
//                  S^T accumulators after exp2 and rounding to the element type.
//   For the second product the 8 keys a lane feeds at k-slot (l/32, t) must be
//   the 8 keys its S^T accumulator holds.  Staging K row `key` into LDS row
//   kappa(key) (kappa swaps bits 2 and 3 of the row index) makes accumulator
//   register j of a 32-key S^T tile hold key 16*(j/8) + 8*(l/32) + j%8, so
//   the keys of PV step c are the contiguous run 16c + 8*(l/32) + 0..7 and the
//   matching V^T operand is one 16-byte LDS read.
//
// Raster variant (no gather or scatter passes): Q, K, V are read and O is
// written in the raster layout [B,S,NH,D] by block index arithmetic.  A
// block's valid tokens, taken in raster order inside its box, lie at token
// offsets from the box origin that depend only on which of the box's three
// extents the grid edge cuts, so each workgroup first tabulates those offsets
// for the 8 possible edge classes in LDS; a sub-tile descriptor then carries
// the block's origin token, class and sub-tile index, and each lane's source
// offset for a copy is one LDS table read.  Pad rows of a partial sub-tile
// re-read a valid row (masked as before).  V stays token-major in LDS (64 key
// rows of 256 B plus a 32-byte pad) and the PV operands are read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes,
// lane i receives element i%4 of the 8-byte rows addressed by lanes
// 4e + i/4 (e = 0..3), so two such reads give a lane the 8 consecutive keys of
// one d column that the V^T layout holds as one 16-byte read.  A 32-lane
// half of such a read covers 4 key rows; so that it touches 8 distinct
// 32-byte bank groups, the MFMA row m of O^T tile dt holds
// d = 64*(m/16) + 16*dt + m%16 (lanes 16..31 read 128 bytes further along
// the row) instead of 32*dt + m.  Rounding and product order are those of the
// blocked kernel: both write identical O.
//
// Online softmax (exact up to rounding): running reference max m and sum l per
// query in fp32, p = exp2(s*log2(e)/sqrt(D) - m*log2(e)/sqrt(D)) on the
// transcendental unit, l summed from the fp32 p, P rounded to bf16 (fp16 for
// fp16 tensors) for the PV product, O rescaled by exp2 of the max change only
// when the max grows by more than 2^8 (so p <= 256).  Padded keys of a partial sub-tile are masked
// to -inf.  A row without blocks leaves l = 0 and writes O = 0, LSE = -inf.

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "attn_common.h"
#include "vsa_internal.h"

// Device scratch of vsa_block_sparse_attn_fwd_noalloc: the row-queue counters,
// claim order and tail-split region of the balanced launch, in a fixed
// library-owned array (one copy per GPU,
// held until the process ends) for callers that cannot allocate.  In host
// code this name only stands for the symbol; kernels receive the device
// address that vsa::noalloc_scratch looks up per device.
static __device__ __align__(256) unsigned char scratch[vsa::kNoAllocScratchBytes];

namespace vsa {
namespace {

using namespace tile;


// A row's CSR entries are flattened, up to kListEntries at a time (768 in the
// 64-token kernel), into a list
// of 64-key sub-tile descriptors in LDS:
//   (64-token chunk index of the sub-tile within its head) << 7 | (valid keys - 1)
// K rows of chunk c start at token row 64c of the head and V^T chunk c is the
// c-th 64-token chunk, so the chunk index addresses both.
constexpr int kListEntries = 1024;

// Raster sub-tile descriptor:
//   origin token of the block << 11 | edge class << 8 | sub-tile << 6 | (valid keys - 1)
// (origin < 2^21 tokens; the host checks it).
constexpr int kRasterVRow = 18;  // raster V tile row: 16 units of data + 2 pad units (288 B)

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (see the header comment for its lane layout).
__device__ inline v4i16 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
}

// Origin token (raster index of the box corner) and edge class of block j:
// bit 2 / 1 / 0 set when the block is the last one along T / H / W.
__device__ inline void block_origin_class(const VsaGeom& g, int j, int& origin, int& cls) {
  const int plane = g.nbh * g.nbw;
  const int it = j / plane;
  const int rem = j - it * plane;
  const int ih = rem / g.nbw;
  const int iw = rem - ih * g.nbw;
  origin = (it * g.bt * g.H + ih * g.bh) * g.W + iw * g.bw;
  cls = (it == g.nbt - 1 ? 4 : 0) | (ih == g.nbh - 1 ? 2 : 0) | (iw == g.nbw - 1 ? 1 : 0);
}

// soff[c*VOL + s]: offset, in 16-byte units of the raster tensor, of the s-th
// valid token of a block of edge class c from its origin token (slots past
// the valid count repeat the last valid token).
template <int VOL>
__device__ inline void build_slot_table(const VsaGeom& g, uint32_t* soff, int tid, int nthreads) {
  for (int idx = tid; idx < 8 * VOL; idx += nthreads) {
    const int c = idx / VOL, s = idx % VOL;
    const int ct = (c & 4) ? g.T - (g.nbt - 1) * g.bt : g.bt;
    const int ch = (c & 2) ? g.H - (g.nbh - 1) * g.bh : g.bh;
    const int cw = (c & 1) ? g.W - (g.nbw - 1) * g.bw : g.bw;
    const int sc = min(s, ct * ch * cw - 1);
    const int dw = sc % cw;
    const int r2 = sc / cw;
    const int dh = r2 % ch;
    const int dt = r2 / ch;
    soff[idx] = ((uint32_t(dt) * uint32_t(g.H) + uint32_t(dh)) * uint32_t(g.W) + uint32_t(dw)) *
                uint32_t(g.heads) * 16u;
  }
}

// Keep the scheduler from moving work across this point: the main loop is
// laid out slot by slot (one MFMA, its operand prefetch and a share of the
// softmax VALU work per slot) and each slot is fenced.
__device__ inline void slot_fence() { __builtin_amdgcn_sched_barrier(0); }
// Materialise a VALU result where it is written in the source (an empty
// volatile asm that reads and writes the register), so that pure arithmetic
// is not sunk towards its first use and stays in its slot.
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Clears the row-queue counters and the tail-split counters of a balanced
// launch (a kernel rather than a memset, so that the launch can be recorded
// into a graph).
__global__ void queue_reset_kernel(unsigned int* queues, unsigned int* flags, int nflags) {
  if (threadIdx.x < 9) queues[threadIdx.x] = 0u;
  for (int x = threadIdx.x; x < nflags; x += blockDim.x) flags[x] = 0u;
}

// Row max over the 16 scores of one tile.
__device__ inline float tile_max1(const f32x16& st) {
  float mx = st[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, st[j]);
  return mx;
}

// Row max over the 32 scores this lane holds.
__device__ inline float tile_max(const f32x16 (&st)[2]) {
  float mx = st[0][0];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[mt][j]);
  return mx;
}

// RASTER = false: q, k, o blocked [B,NH,Npad,D], v blocked-V^T.
// RASTER = true: q, k, v, o raster [B,S,NH,D]; with `gate` (raster) the
// output is O + gate * oc[block] (oc fp32 [B,NH,nb,D]), as the gated scatter.
// NQ: query row groups of 32 per block (block volume 32*NQ); NW: waves, NQ,
// or 2*NQ for 64-token blocks whose two groups are each split by key halves.
template <int NW, int NQ, bool F16, bool RASTER>
__global__ __launch_bounds__(NW * 64, NW == 2 * NQ ? 2 : 1) void attn_fwd_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int uniform_k,
    int64_t nnz, uint4* __restrict__ o, float* __restrict__ lse, const uint4* __restrict__ gate,
    const float* __restrict__ oc, unsigned int* __restrict__ queues,
    const int32_t* __restrict__ order, VsaGeom g, float scale_log2, float scale, TailSplit ts) {
  static_assert(NW == NQ || (NQ == 2 && NW == 4), "waves: one per query group, or 4 for 2 groups");
  static_assert(NW * 32 * kORow <= 2 * (kKUnits + kVUnits) && 8 * 32 * kORow <= 4 * kKUnits,
                "O staging must fit in LDS");
  const float rescale_thr = 8.0f / scale_log2;  // raw-score growth that triggers a rescale
  // Sub-tile buffers of the 4- and 6-wave kernels.  K runs one sub-tile
  // ahead of V: while sub-tile n is finished, K buffer (n+1)%2 holds K_{n+1}
  // (read) and K buffer n%2 receives K_{n+2}; V buffer n%2 holds V_n (read)
  // and V buffer (n+1)%2 receives V_{n+1}.  Four separate arrays let the
  // compiler see that the in-flight copies never alias the buffers being read.
  // The 8-wave kernel's alternating pipeline (below) keeps rings of four K
  // and three V sub-tiles instead.
  constexpr bool kPP = NW == 8 && !RASTER;
  __shared__ __align__(16) uint4 kbuf0[kPP ? 1 : kKUnits];
  __shared__ __align__(16) uint4 kbuf1[kPP ? 1 : kKUnits];
  __shared__ __align__(16) uint4 vbuf0[kPP ? 1 : kVUnits];
  __shared__ __align__(16) uint4 vbuf1[kPP ? 1 : kVUnits];
  __shared__ __align__(16) uint4 kring[kPP ? 4 * kKUnits : 1];
  __shared__ __align__(16) uint4 vring[kPP ? 3 * kVUnits : 1];
  // sub-tile descriptor list of the current pass over the row, and the
  // per-entry scan that places each entry's descriptors
  constexpr int kThreads = NW * 64;
  // Two workgroups of 64-token blocks share a CU only if each holds at most
  // half of its 160 KB of LDS; their list passes are shorter to leave room
  // for the raster slot table.
  constexpr int kList = NQ == 2 ? 768 : kListEntries;
  constexpr int kListTiles = kList * (32 * NQ / kKvChunk);
  __shared__ int tlist[kListTiles];
  __shared__ int escan[kList];
  __shared__ int ntiles_sh;
  constexpr int kVol = 32 * NQ;
  __shared__ uint32_t soff[RASTER ? 8 * kVol : 1];
  static_assert(NQ != 2 || 16 * 2 * (kKUnits + kVUnits) + 4 * (kListTiles + kList) +
                               4 * (RASTER ? 8 * kVol : 1) + 64 <= 160 * 1024 / 2,
                "two workgroups of 64-token blocks must fit in one CU's LDS");

  const int64_t nrows = int64_t(g.batch) * g.heads * g.nb;
  // The row: fixed by the workgroup index (XCD-aware order), or, with
  // `queues`, claimed at start-up (claim_row); a workgroup that finds every
  // row taken leaves at once (workgroup-uniform, before any other barrier).
  __shared__ int64_t row_sh;
  __shared__ int part_sh;
  const uint32_t tail_split = queues == nullptr ? 0u : uint32_t(ts.per_queue);
  const int64_t r = queues == nullptr ? xcd_remap(blockIdx.x, nrows)
                    : (row_ptr == nullptr && g.head_interleave)
                        ? claim_row_strided(queues, nrows, g, &row_sh, tail_split, &part_sh)
                        : claim_row(queues, nrows, g, &row_sh, order, tail_split, &part_sh);
  if (r < 0) return;
  // -1: the whole row; else this workgroup computes half (part & 1) of the
  // row's entries for split slot part / 2 (workgroup-uniform)
  const int part = tail_split != 0 ? part_sh : -1;
  const int i = int(r % g.nb);
  const int64_t bh = r / g.nb;
  const int cq = block_count(g, i);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: lives in an SGPR
  const int lane = tid % 64;
  const int half = lane / 32;
  const int l32 = lane & 31;
  // Query row groups.  Normally wave w owns rows 32w .. 32w+31.  The 8-wave
  // kernel runs the alternating pipeline below, in which waves w and w+4
  // (always on the same SIMD) take turns on the matrix cores, so each SIMD
  // needs work for both: with 5 or 6 groups holding valid rows (a block cut
  // by the grid edge), waves 4..7 share the last groups by keys: waves 4 and
  // 6 take group 4, waves 5 and 7 group 5; with at most 4 groups, waves w and
  // w+4 share group w.  In such a pair the first wave takes keys 0..31 of
  // every sub-tile and the second keys 32..63, each with its own online
  // softmax, and the pair merges before the epilogue.
  // With 4 waves on a 64-token block (NW = 2*NQ) every group is split:
  // waves 0 and 2 take group 0, waves 1 and 3 group 1, waves 0 and 1 keys
  // 0..31 and waves 2 and 3 keys 32..63.
  const int ngroups = (cq + 31) / 32;
  constexpr bool kAllSplit = NW == 2 * NQ;
  const bool split = kAllSplit || (NW == 8 && (ngroups == 5 || ngroups == 6));  // wg-uniform
  const bool split4 = kPP && ngroups <= 4;                                      // wg-uniform
  const int qgroup = kAllSplit ? wave % NQ
                     : split4  ? wave & 3
                               : (split && wave >= 4 ? 4 + (wave & 1) : wave);
  const int khalf = kAllSplit ? wave / NQ
                    : split4  ? wave >> 2
                              : (split && wave >= 4 ? (wave >> 1) & 1 : -1);  // -1: all 64 keys
  const int qrow = qgroup * 32 + l32;    // this lane's query row inside the block
  const bool active = qgroup * 32 < cq;  // wave-uniform

  int64_t beg, end;
  if (row_ptr != nullptr) {
    beg = min(max(int64_t(row_ptr[r]), int64_t(0)), nnz);
    end = min(max(int64_t(row_ptr[r + 1]), beg), nnz);
  } else {
    beg = r * uniform_k;
    end = beg + uniform_k;
  }
  if (part >= 0) {
    // a half of a split row: the first or the second half of its entries
    const int64_t mid = beg + (end - beg) / 2;
    if (part & 1) beg = mid;
    else end = mid;
  }
  const int32_t* rcol = col + beg;
  const int len = int(end - beg);

  const int64_t qk_row0 = bh * g.npad + int64_t(i) * g.vol;  // first token row of block i
  // raster: first unit of head h in batch b, the token stride, block i's origin and class
  int64_t head0 = 0, rs = 0;
  int origin_i = 0, cls_i = 0;
  if constexpr (RASTER) {
    head0 = ((bh / g.heads) * g.S * g.heads + bh % g.heads) * 16;
    rs = int64_t(g.heads) * 16;
    block_origin_class(g, i, origin_i, cls_i);
    build_slot_table<kVol>(g, soff, tid, kThreads);
    __syncthreads();
  }
  ev8 qf[8];
  if (active) {
    const uint4* qsrc;
    if constexpr (RASTER)
      qsrc = q + head0 + origin_i * rs + soff[cls_i * kVol + min(qrow, cq - 1)];
    else
      qsrc = q + (qk_row0 + qrow) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_ev8(qsrc[2 * s + half]);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[dt][j] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint4* const kbase = RASTER ? k + head0 : k + bh * g.npad * 16;
  const uint4* const vbase = RASTER ? v + head0 : v + bh * (g.npad / kKvChunk) * kUnits;
  const int chunks_per_block = g.vol / kKvChunk;
  // Copy x of a sub-tile moves LDS chunk wave + x*NW (64 consecutive 16-byte
  // units of the padded buffer); koff/voff are this lane's source offsets
  // inside the sub-tile, the same for every sub-tile.  Chunk positions past
  // the buffer belong to copies that the lane predicate switches off.
  constexpr int kMaxK = (kKChunks + NW - 1) / NW, kMaxV = (kVChunks + NW - 1) / NW;
  // With 8 or 6 waves each issues at most 3 + 3 copies per sub-tile and they
  // are placed inside the MFMA slots; with fewer waves (up to 9 + 9 copies
  // each) predicated copies inside the slots make the compiler duplicate the
  // slot code many times over, so those copies go at the top of the step.
  constexpr bool kSlotCopies = kMaxK + kMaxV <= 6;
  // Blocked: koff/voff are the lane's source offsets inside a sub-tile.
  // Raster: krow/vrow are the sub-tile rows (keys) the lane copies and
  // kun/vun the 16-byte units inside the token row; the row's offset comes
  // from the slot table.  The pad units of a row re-read units of that row.
  constexpr int kVRowX = RASTER ? kRasterVRow : kVRow;
  uint32_t koff[kMaxK], voff[kMaxV];
  int krow[kMaxK], vrow[kMaxV];
#pragma unroll
  for (int x = 0; x < kMaxK; ++x) {
    const int pos = min((wave + x * NW) * 64 + lane, kKUnits - 1);
    const int row = pos / kKRow, unit = pos % kKRow;
    koff[x] = RASTER ? (unit < 16 ? unit : 0) : kappa(row) * 16 + (unit < 16 ? unit : 0);
    krow[x] = kappa(row);
  }
#pragma unroll
  for (int x = 0; x < kMaxV; ++x) {
    const int pos = min((wave + x * NW) * 64 + lane, kVUnits - 1);
    const int row = pos / kVRowX, unit = pos % kVRowX;
    if constexpr (RASTER) voff[x] = unit < 16 ? unit : unit - 16;
    else voff[x] = row * 8 + (unit < 8 ? unit : 0);
    vrow[x] = row;
  }
  auto src_of = [&](const uint4* base, int desc) {
    if constexpr (RASTER) return base + int64_t(uint32_t(desc) >> 11) * rs;
    else return base + int64_t(desc >> 7) * kUnits;
  };
  // source offsets of this lane's copies of the sub-tile `desc`
  auto k_offsets = [&](int desc, uint32_t (&ko)[kMaxK]) {
    const int tb = ((desc >> 8) & 7) * kVol + ((desc >> 6) & 3) * 64;
#pragma unroll
    for (int x = 0; x < kMaxK; ++x) ko[x] = RASTER ? soff[tb + krow[x]] + koff[x] : koff[x];
  };
  auto v_offsets = [&](int desc, uint32_t (&vo)[kMaxV]) {
    const int tb = ((desc >> 8) & 7) * kVol + ((desc >> 6) & 3) * 64;
#pragma unroll
    for (int x = 0; x < kMaxV; ++x) vo[x] = RASTER ? soff[tb + vrow[x]] + voff[x] : voff[x];
  };
  // The predicate is wave-uniform (whether this wave owns chunk x of the
  // sub-tile); the slot fences keep each copy in its slot either way.
  auto copy_k = [&](const uint4* src, uint32_t off, int x, uint4* dst) {
    if (tid / 64 + x * NW < kKChunks) wave_copy_to_lds(src, off, dst + (wave + x * NW) * 64);
  };
  auto copy_v = [&](const uint4* src, uint32_t off, int x, uint4* dst) {
    if (tid / 64 + x * NW < kVChunks) wave_copy_to_lds(src, off, dst + (wave + x * NW) * 64);
  };
  auto load_k = [&](int desc, uint4* dst) {
    uint32_t ko[kMaxK];
    k_offsets(desc, ko);
#pragma unroll
    for (int x = 0; x < kMaxK; ++x) copy_k(src_of(kbase, desc), ko[x], x, dst);
  };
  auto load_v = [&](int desc, uint4* dst) {
    uint32_t vo[kMaxV];
    v_offsets(desc, vo);
#pragma unroll
    for (int x = 0; x < kMaxV; ++x) copy_v(src_of(vbase, desc), vo[x], x, dst);
  };
  // the same copies issued from inline asm (wave_copy_to_lds_async)
  auto load_k_async = [&](int desc, uint4* dst) {
    uint32_t ko[kMaxK];
    k_offsets(desc, ko);
#pragma unroll
    for (int x = 0; x < kMaxK; ++x)
      if (tid / 64 + x * NW < kKChunks)
        wave_copy_to_lds_async(src_of(kbase, desc), ko[x] * 16u,
                               lds_addr(dst + (wave + x * NW) * 64));
  };
  auto load_v_async = [&](int desc, uint4* dst) {
    uint32_t vo[kMaxV];
    v_offsets(desc, vo);
#pragma unroll
    for (int x = 0; x < kMaxV; ++x)
      if (tid / 64 + x * NW < kVChunks)
        wave_copy_to_lds_async(src_of(vbase, desc), vo[x] * 16u,
                               lds_addr(dst + (wave + x * NW) * 64));
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // per-lane operand bases: K row l32 (+ half unit), V^T row l32 (+ half unit)
  const int kread = l32 * kKRow + half;
  const int vread = l32 * kVRow + half;
  // raster: byte offset of this lane's transposing V read: key row
  // 8*half + e (e = (lane%16)/4), d column 64*((lane/16)%2) + 4*(lane%4)
  const int vtr = (8 * half + (lane & 15) / 4) * (kRasterVRow * 16) +
                  (64 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  // operand bases of a key-half wave: keys 32*kh .. 32*kh+31 of each sub-tile
  const int kh = khalf > 0 ? 1 : 0;
  const int kread_h = kread + kh * 32 * kKRow;
  const int vread_h = vread + kh * 4;
  const int vtr_h = vtr + kh * 32 * (kRasterVRow * 16);

  // ---- Alternating pipeline of the 8-wave kernel.  Waves 0..3 (group A)
  // and 4..7 (group B) put one wave on each SIMD each and take turns: while
  // one wave of a SIMD runs the matrix phase of a sub-tile (M: S_{n+1} =
  // K_{n+1} Q^T and O^T += V^T_n P^T_n, MFMAs and their LDS operand reads) the
  // other runs its softmax phase (S: mask, row max exchange, rescale,
  // exponentials, row sums, rounding of P, and the wave's share of the
  // global->LDS copies).  A wave issues in order, so with both kinds of work
  // interleaved in every wave's stream the older wave of a SIMD held the
  // matrix cores while the younger one waited behind its own MFMAs with its
  // softmax work unissued.
  //   Phases are separated by workgroup barriers.  Group A runs QK_0 | S_0 |
  // M_0 | S_1 | M_1 | ..., group B the same one phase later: in phase 2n
  // group A runs M_n while group B runs S_n, in phase 2n+1 A runs S_{n+1}
  // while B runs M_n.  K_j lives in K ring slot j % 4, V_j in V ring slot j % 3.
  // In S_j group A copies K_{j+3} (into the slot of K_{j-1}, last read by
  // M_{j-2}) and group B copies V_{j+2} (into the slot of V_{j-1}, last read
  // by M_{j-1}); at the end of its next M phase each wave waits for all but
  // the copies of its latest S phase, so a copy has three phases to land
  // before the barrier ahead of its first reader (the S phase that reads the
  // first K operands of the M phase using it, or that M phase for V).
  // The copies are issued from inline asm: their destinations are computed
  // at run time, and the compiler, unable to place them, would otherwise
  // wait for all of them before every LDS read.
  auto pp_pipeline = [&](auto hv, auto gbt, auto comp, int T, auto desc_at)
      __attribute__((always_inline)) {
    constexpr bool HV = decltype(hv)::value;          // key-half wave
    constexpr bool GB = decltype(gbt)::value;         // group B (waves 4..7)
    constexpr bool kCompute = decltype(comp)::value;  // the wave holds query rows
    static_assert(!RASTER, "the alternating pipeline serves the blocked layout");
    constexpr int NQK = HV ? 8 : 16;                  // QK^T MFMAs per sub-tile
    constexpr int NPV = HV ? 8 : 16;                  // PV MFMAs per sub-tile
    constexpr int NE = HV ? 8 : 16;                   // exponential pairs per sub-tile
    // group A copies the 17 chunks of a K sub-tile, group B the 18 of a V
    // sub-tile; wave gw of a group copies chunks gw, gw+4, gw+8, ...
    constexpr int kChunks = GB ? kVChunks : kKChunks;
    constexpr int NCP = (kChunks + 3) / 4;
    const int gw = wave & 3;
    const bool last_copy = gw + 4 * (NCP - 1) < kChunks;  // wave-uniform: NCP copies, else NCP-1
    f32x16 sacc[2];
    float mx_pre = -INFINITY;
    uint32_t pw[4][4];
    ev8 op[8];  // operand ring of the M phase
    constexpr int kPre = 4;  // operand reads in flight ahead of their MFMA
    // this lane's source byte offsets within a sub-tile
    uint32_t cofs[NCP];
#pragma unroll
    for (int x = 0; x < NCP; ++x) {
      const int c = min(gw + 4 * x, kChunks - 1);
      const int pos = c * 64 + lane;
      if constexpr (!GB) {
        const int row = pos / kKRow, unit = pos % kKRow;
        cofs[x] = (kappa(row) * 16 + (unit < 16 ? unit : 0)) * 16;
      } else {
        const int row = pos / kVRow, unit = pos % kVRow;
        cofs[x] = (row * 8 + (unit < 8 ? unit : 0)) * 16;
      }
    }
    constexpr uint32_t kSlotBytes = (GB ? kVUnits : kKUnits) * 16;
    const uint32_t ring0 = lds_addr(GB ? vring : kring) + uint32_t(gw) * 1024u;
    // copy x of this wave: its chunk of sub-tile `desc` into ring slot `slot`
    auto copy_one = [&](int x, const char* src, uint32_t dst) __attribute__((always_inline)) {
      if (x < NCP - 1 || last_copy) wave_copy_to_lds_async(src, cofs[x], dst + uint32_t(x) * 4096u);
    };
    // all but this wave's latest batch of copies have landed
    auto wait_older = [&]() __attribute__((always_inline)) {
      if (last_copy) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCP) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCP - 1) : "memory");
    };
    // Phase barrier.  A fence would make the compiler wait for every load in
    // flight; an empty asm with a memory clobber keeps it from moving LDS
    // accesses across the barrier instead.  No LDS read of a wave can still
    // be pending on a slot that a copy issued after the barrier overwrites:
    // every M-phase read feeds an MFMA of the same phase, and the reads an S
    // phase leaves in flight (the next M phase's first K operands, the
    // descriptors) address slots and lists that stay untouched for several
    // phases.
    auto barrier = []() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    };
    // operand of M-phase slot s: K rows for the QK^T slots, V^T rows for PV
    auto operand = [&](const uint4* kn, const uint4* vn, int s) __attribute__((always_inline)) -> ev8 {
      if (s < NQK) {
        if constexpr (HV) return as_ev8(kn[kread_h + 2 * s]);
        else return as_ev8(kn[kread + (s % 2) * 32 * kKRow + 2 * (s / 2)]);
      }
      const int w = s - NQK, cc = w / 4, dt = w % 4;
      return as_ev8(vn[(HV ? vread_h : vread) + dt * 32 * kVRow + 2 * cc]);
    };
    // M phase: S_{n+1} = K_{n+1} Q^T into sacc (kn) and, with PV, O^T += V^T_n
    // P^T_n (vn, pw).  op[0..kPre-1] hold the operands of the first slots.  The row max
    // of the new scores is taken in the last slots, after its MFMAs.
    auto m_phase = [&](const uint4* kn, const uint4* vn, auto withpv) __attribute__((always_inline)) {
      constexpr bool PV = decltype(withpv)::value;
      constexpr int NS = PV ? NQK + NPV : NQK;
      constexpr int MX0 = NS - (HV ? 4 : 8);  // first slot of the row max
#pragma unroll
      for (int mt = 0; mt < (HV ? 1 : 2); ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[mt][j] = 0.f;
      float mxn = -INFINITY;
      slot_fence();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // one operand read per slot, kPre slots ahead, so that the wave keeps
        // about kPre reads in flight instead of bursts of four
        if (s + kPre < NS) op[(s + kPre) % 8] = operand(kn, vn, s + kPre);
        if (s < NQK) {
          if constexpr (HV) sacc[0] = mfma_32x32x16<F16>(op[s % 8], qf[s], sacc[0]);
          else sacc[s % 2] = mfma_32x32x16<F16>(op[s % 8], qf[s / 2], sacc[s % 2]);
        } else {
          const int w = s - NQK, cc = w / 4, dt = w % 4;
          const ev8 pb =
              __builtin_bit_cast(ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2], pw[cc][3]));
          oacc[dt] = mfma_32x32x16<F16>(op[s % 8], pb, oacc[dt]);
        }
        if (PV && s >= MX0) {
          const int mt = HV ? 0 : (s - MX0) / 4, j0 = ((s - MX0) % 4) * 4;
          mxn = fmaxf(fmaxf(mxn, sacc[mt][j0]), sacc[mt][j0 + 1]);
          mxn = fmaxf(fmaxf(mxn, sacc[mt][j0 + 2]), sacc[mt][j0 + 3]);
          pin(mxn);
        }
        slot_fence();
      }
      if constexpr (!PV) mxn = HV ? tile_max1(sacc[0]) : tile_max(sacc);
      // row max including the partner lane's keys (l ^ 32), taken here so that
      // its latency overlaps the last MFMAs instead of opening the S phase
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mxn), __float_as_uint(mxn),
                                                       false, false);
      mx_pre = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    // S phase of sub-tile j (descriptor dj, scores in sacc): P_j into pw, the
    // running max / sum updated; kpre holds K_{j+1}, whose first operands the
    // next M phase reads (issued last).  cp(e) issues the copies placed after pair e and
    // tells whether there were any.
    auto s_phase = [&](int dj, const uint4* kpre, auto&& cp) __attribute__((always_inline)) {
      float mx = mx_pre;  // the row max over both lane halves (unmasked)
      const int valid = (dj & 127) + 1;
      if (valid < kKvChunk) {
        // key of register j: (32 mt or 32 kh) + 16 (j/8) + 8 half + j%8; the
        // comparison is against valid - 8 half - 32 kh so that every key
        // offset is an immediate
        const int vh = valid - 8 * half - (HV ? 32 * kh : 0);
#pragma unroll
        for (int mt = 0; mt < (HV ? 1 : 2); ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if ((HV ? 0 : mt * 32) + 16 * (j / 8) + (j % 8) >= vh) sacc[mt][j] = -INFINITY;
        mx = HV ? tile_max1(sacc[0]) : tile_max(sacc);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      if (__ballot(mx > m_run + rescale_thr) != 0) {  // wave-uniform
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        m_run = m_new;
        l_run *= alpha;
        // in place: O keeps its registers through the (rare) rescale
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float t = oacc[dt][j];
            asm volatile("v_mul_f32 %0, %0, %1" : "+v"(t) : "v"(alpha));
            oacc[dt][j] = t;
          }
      }
      // a key half may have seen only masked keys so far (m_run = -inf); any
      // finite reference then gives p = 0 for them
      const float mb = (HV && m_run == -INFINITY) ? 0.f : m_run * scale_log2;
      // four row-sum accumulators (pairs e % 2 and both lanes of a pair), so
      // the additions do not form one long dependent chain
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int cc = e / 4, t = 2 * (e % 4);
        const float s0 = HV ? sacc[0][8 * cc + t] : sacc[cc / 2][8 * (cc % 2) + t];
        const float s1 = HV ? sacc[0][8 * cc + t + 1] : sacc[cc / 2][8 * (cc % 2) + t + 1];
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s0, scale_log2, -mb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s1, scale_log2, -mb));
        rs[2 * (e % 2)] += p0;
        rs[2 * (e % 2) + 1] += p1;
        pw[cc][t / 2] = pack2<F16>(p0, p1);
        // the wave's copies stay spread over the phase (issued together, the
        // four SIMDs' copies queue behind each other at the CU's vector
        // memory unit); between copies the scheduler may overlap the pairs
        if (cp(e)) {
          pin(rs[2 * (e % 2)]);
          pin(rs[2 * (e % 2) + 1]);
          pin(pw[cc][t / 2]);
          slot_fence();
        }
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      // the next M phase's first operands, left in flight across the barrier
#pragma unroll
      for (int x = 0; x < kPre; ++x) op[x] = operand(kpre, nullptr, x);
    };
    auto kslot = [&](int sl) __attribute__((always_inline)) { return kring + sl * kKUnits; };
    auto vslot = [&](int sl) __attribute__((always_inline)) { return vring + sl * kVUnits; };
    // S phase of sub-tile j (descriptor dj): the softmax (with rows) and this
    // wave's copies of sub-tile dc (group A: K_{j+3} into K slot cslot; group
    // B: V_{j+2} into V slot cslot)
    auto s_full = [&](int dj, int dc, int kpre_slot, int cslot) __attribute__((always_inline)) {
      const char* const src = reinterpret_cast<const char*>(src_of(GB ? vbase : kbase, dc));
      const uint32_t dst = ring0 + uint32_t(cslot) * kSlotBytes;
      if constexpr (kCompute) {
        // copy x after exponential pair x * NE / NCP
        s_phase(dj, kslot(kpre_slot), [&](int e) __attribute__((always_inline)) {
          bool any = false;
#pragma unroll
          for (int x = 0; x < NCP; ++x)
            if (e == (x * NE) / NCP) {
              copy_one(x, src, dst);
              any = true;
            }
          return any;
        });
      } else {
#pragma unroll
        for (int x = 0; x < NCP; ++x) copy_one(x, src, dst);
      }
    };
    auto rfl = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };

    // prologue: K_0, K_1, K_2 and V_0, V_1 by all waves
    const int d0 = __builtin_amdgcn_readfirstlane(desc_at(0));
    load_k_async(d0, kslot(0));
    load_k_async(__builtin_amdgcn_readfirstlane(desc_at(1)), kslot(1));
    load_k_async(__builtin_amdgcn_readfirstlane(desc_at(2)), kslot(2));
    load_v_async(d0, vslot(0));
    load_v_async(__builtin_amdgcn_readfirstlane(desc_at(1)), vslot(1));
    wait_loads();
    barrier();
    auto qk0 = [&]() __attribute__((always_inline)) {
      if constexpr (kCompute) {
#pragma unroll
        for (int x = 0; x < kPre; ++x) op[x] = operand(kslot(0), nullptr, x);
        m_phase(kslot(0), nullptr, std::false_type());
      }
    };
    if constexpr (!GB) {
      qk0();  // phase -2 (group B: nothing)
      barrier();
      s_full(d0, rfl(desc_at(3)), 1, 3);  // phase -1: S_0, K_3 into slot 3 (group B: QK_0)
      barrier();
    } else {
      barrier();  // phase -2
      qk0();      // phase -1
      barrier();
      s_full(d0, rfl(desc_at(2)), 1, 2);  // phase 0: S_0, V_2 into slot 2 (group A: M_0)
      barrier();
    }
    // iteration n: M_n (K_{n+1} in slot k1, V_n in slot v0), the wait for
    // this wave's copies of S_{n-1} (those of S_n stay in flight), barrier,
    // S_{n+1} (first operands of K_{n+2}; group A copies K_{n+4} into the slot
    // of K_n, group B V_{n+3} into the slot of V_n), barrier.  A copy thus has
    // three phases to land before the barrier ahead of its first reader.
    int k1 = 1, v0 = 0;
    for (int n = 0; n < T; ++n) {
      // descriptors of S_{n+1}, read before M_n so that it hides their latency
      const int dj = desc_at(n + 1), dc = desc_at(GB ? n + 3 : n + 4);
      if constexpr (kCompute) m_phase(kslot(k1), vslot(v0), std::true_type());
      wait_older();
      barrier();
      if (n + 1 < T) s_full(rfl(dj), rfl(dc), (k1 + 1) & 3, GB ? v0 : (k1 + 3) & 3);
      barrier();
      k1 = (k1 + 1) & 3;
      v0 = v0 == 2 ? 0 : v0 + 1;
    }
    // group A's last phase: group B runs M_{T-1}
    if constexpr (!GB) barrier();
    wait_loads();
    __syncthreads();
  };

  // Flatten row entries e0 .. e0+m-1 (m = min(kList, len - e0)) into the
  // sub-tile list: per-entry sub-tile counts, an exclusive scan of them, then
  // the descriptors.  Returns the number of sub-tiles (wave-uniform).
  auto build_list = [&](int e0) __attribute__((always_inline)) -> int {
    const int m = min(kList, len - e0);
    for (int e = tid; e < m; e += kThreads) {
      const int j = rcol[e0 + e];
      escan[e] = (j >= 0 && j < g.nb) ? (block_count(g, j) + kKvChunk - 1) / kKvChunk : 0;
    }
    __syncthreads();
    if (wave == 0) {
      constexpr int kPerLane = kList / 64;
      int loc[kPerLane];
      int sum = 0;
#pragma unroll
      for (int x = 0; x < kPerLane; ++x) {
        const int e = lane * kPerLane + x;
        loc[x] = sum;
        sum += e < m ? escan[e] : 0;
      }
      int incl = sum;
#pragma unroll
      for (int d = 1; d < 64; d *= 2) {
        const int up = __shfl_up(incl, d);
        if (lane >= d) incl += up;
      }
      const int base = incl - sum;
#pragma unroll
      for (int x = 0; x < kPerLane; ++x) {
        const int e = lane * kPerLane + x;
        if (e < m) escan[e] = base + loc[x];
      }
      if (lane == 63) ntiles_sh = incl;
    }
    __syncthreads();
    for (int e = tid; e < m; e += kThreads) {
      const int j = rcol[e0 + e];
      if (j >= 0 && j < g.nb) {
        const int cj = block_count(g, j);
        const int off = escan[e];
        if constexpr (RASTER) {
          int origin, cls;
          block_origin_class(g, j, origin, cls);
          for (int sub = 0; sub * kKvChunk < cj; ++sub)
            tlist[off + sub] = int((uint32_t(origin) << 11) | uint32_t(cls << 8) |
                                   uint32_t(sub << 6) |
                                   uint32_t(min(kKvChunk, cj - sub * kKvChunk) - 1));
        } else {
          for (int sub = 0; sub * kKvChunk < cj; ++sub)
            tlist[off + sub] =
                ((j * chunks_per_block + sub) << 7) | (min(kKvChunk, cj - sub * kKvChunk) - 1);
        }
      }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(ntiles_sh);
  };
  // The passes over the row (list building, prologue, pipelined steps) of
  // the 4- and 6-wave kernels are compiled twice, for full waves (HV = false)
  // and for key-half waves, each with its own register allocation; a wave
  // runs one of them.
  auto passes = [&](auto hv) __attribute__((always_inline)) {
  constexpr bool HV = decltype(hv)::value;
  f32x16 sa[2], sb[2];
  float mx_pre = -INFINITY;  // unmasked row max of the scores of sub-tile n

  for (int e0 = 0; e0 < len; e0 += kList) {
    const int T = build_list(e0);
    if (T == 0) continue;
    // descriptor of sub-tile n; past the end it repeats the last one, whose
    // copies then land in a buffer that is not read again
    auto desc_at = [&](int n) { return tlist[min(n, T - 1)]; };

    int n = 0;
    int d0 = __builtin_amdgcn_readfirstlane(desc_at(0));
    int d1 = __builtin_amdgcn_readfirstlane(desc_at(1));
    int d2 = __builtin_amdgcn_readfirstlane(desc_at(2));
    load_k(d0, kbuf0);
    load_v(d0, vbuf0);
    load_k(d1, kbuf1);
    wait_loads();
    __syncthreads();
    if (active && !HV) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) sa[mt][j] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          sa[mt] = mfma_32x32x16<F16>(as_ev8(kbuf0[kread + mt * 32 * kKRow + 2 * s]), qf[s],
                                      sa[mt]);
      mx_pre = tile_max(sa);
    } else if (active) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sa[0][j] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        sa[0] = mfma_32x32x16<F16>(as_ev8(kbuf0[kread_h + 2 * s]), qf[s], sa[0]);
      mx_pre = tile_max1(sa[0]);
    }
    // the first step copies K_2 into kbuf0: every wave must be done with K_0
    __syncthreads();

    // The step of a key-half wave: the same pipeline on one 32-key S^T tile
    // per sub-tile, laid out in 16 slots (8 QK^T, then 8 PV).
    auto half_body = [&](f32x16& cur, f32x16& nxt, const uint4* kn, uint4* kw, const uint4* vn,
                         uint4* vw, const uint4* sk, const uint4* sv, const uint32_t (&ko)[kMaxK],
                         const uint32_t (&vo)[kMaxV]) __attribute__((always_inline)) {
      // first K operands before the row-max exchange, as in the full step
      ev8 opk[8], opv[8];
      auto read_k = [&](int u) { opk[u % 8] = as_ev8(kn[kread_h + 2 * u]); };
#pragma unroll
      for (int u = 0; u < 4; ++u) read_k(u);
      float mx = mx_pre;
      const int valid = (d0 & (RASTER ? 63 : 127)) + 1;
      if (valid < kKvChunk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kh * 32 + 16 * (j / 8) + 8 * half + (j % 8);
          if (key >= valid) cur[j] = -INFINITY;
        }
        mx = tile_max1(cur);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      if (__ballot(mx > m_run + rescale_thr) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
      }
      // A key half may see only masked keys for a while (m_run = -inf); any
      // finite reference then gives p = 0 for them.
      const float mb = m_run == -INFINITY ? 0.f : m_run * scale_log2;
      float rs0 = 0.f, rs1 = 0.f;
      uint32_t pw[2][4];
      float mxn = -INFINITY;
      auto read_v = [&](int w) {  // PV slot w: keys 32*kh + 16*(w/4) + ..., d tile w%4
        if constexpr (RASTER) {
          const char* bp = reinterpret_cast<const char*>(vn) + vtr_h +
                           (16 * (w / 4)) * (kRasterVRow * 16) + 32 * (w % 4);
          const v4i16 lo = lds_read_tr16(bp);
          const v4i16 hi = lds_read_tr16(bp + 4 * (kRasterVRow * 16));
          opv[w % 8] = __builtin_bit_cast(ev8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          opv[w % 8] = as_ev8(vn[vread_h + (w % 4) * 32 * kVRow + 2 * (w / 4)]);
        }
      };
#pragma unroll
      for (int j = 0; j < 16; ++j) nxt[j] = 0.f;
      slot_fence();
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if constexpr (kSlotCopies) {
#pragma unroll
          for (int x = 0; x < kMaxK; ++x)
            if (u == 1 + (x * 8) / kMaxK) copy_k(sk, ko[x], x, kw);
#pragma unroll
          for (int x = 0; x < kMaxV; ++x)
            if (u == 9 + (x * 8) / kMaxV) copy_v(sv, vo[x], x, vw);
        }
        if (u < 8) {
          if (u % 4 == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              if (u + 4 < 8) read_k(u + 4 + x);
              else read_v(x);
            }
          }
          nxt = mfma_32x32x16<F16>(opk[u % 8], qf[u], nxt);
          // exponential pair u: keys 2(u%4), 2(u%4)+1 of PV step u/4
          const int cc = u / 4, t = 2 * (u % 4);
          float p0 = __builtin_amdgcn_exp2f(fmaf(cur[8 * cc + t], scale_log2, -mb));
          float p1 = __builtin_amdgcn_exp2f(fmaf(cur[8 * cc + t + 1], scale_log2, -mb));
          rs0 += p0;
          rs1 += p1;
          pw[cc][t / 2] = pack2<F16>(p0, p1);
          pin(rs0);
          pin(rs1);
          pin(pw[cc][t / 2]);
        } else {
          const int w = u - 8, cc = w / 4, dt = w % 4;
          if (w == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x) read_v(4 + x);
          }
          const ev8 pb = __builtin_bit_cast(
              ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2], pw[cc][3]));
          oacc[dt] = mfma_32x32x16<F16>(opv[w % 8], pb, oacc[dt]);
          if (u >= 12) {
            const int j0 = (u - 12) * 4;
            mxn = fmaxf(fmaxf(mxn, nxt[j0]), nxt[j0 + 1]);
            mxn = fmaxf(fmaxf(mxn, nxt[j0 + 2]), nxt[j0 + 3]);
            pin(mxn);
          }
        }
        slot_fence();
      }
      l_run += rs0 + rs1;
      mx_pre = mxn;
    };

    // Finish sub-tile n (scores in `cur`) and compute the scores of n+1 into
    // `nxt`.  kn: K buffer holding K_{n+1}; kw: K buffer receiving K_{n+2};
    // vn: V buffer holding V_n; vw: V buffer receiving V_{n+1}.
    auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const uint4* kn, uint4* kw,
                    const uint4* vn, uint4* vw) __attribute__((always_inline)) {
      const uint4* const sk = src_of(kbase, d2);
      const uint4* const sv = src_of(vbase, d1);
      const int d3 = desc_at(n + 3);  // LDS read; made uniform after the barrier
      uint32_t ko[kMaxK], vo[kMaxV];
      if constexpr (!kSlotCopies) {
        load_k(d2, kw);
        load_v(d1, vw);
      } else {
        k_offsets(d2, ko);
        v_offsets(d1, vo);
      }
      if (HV && active) {
        half_body(cur[0], nxt[0], kn, kw, vn, vw, sk, sv, ko, vo);
      } else if (!HV && active) {
        // The first K operands of the QK^T slots are read before the row-max
        // exchange and the rescale test, so the LDS latency after the
        // barrier overlaps that chain.
        ev8 opk[8], opv[8];
        auto read_k = [&](int u) {  // operand of QK slot u
          opk[u % 8] = as_ev8(kn[kread + (u % 2) * 32 * kKRow + 2 * (u / 2)]);
        };
#pragma unroll
        for (int u = 0; u < 4; ++u) read_k(u);
        float mx = mx_pre;
        // mask keys past the block's valid count (only in its last sub-tile)
        const int valid = (d0 & (RASTER ? 63 : 127)) + 1;
        if (valid < kKvChunk) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int key = mt * 32 + 16 * (j / 8) + 8 * half + (j % 8);
              if (key >= valid) cur[mt][j] = -INFINITY;
            }
          mx = tile_max(cur);
        }
        // row max including the partner lane's keys (l ^ 32)
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        // Lazy rescale: the reference max m_run only moves (and O, l are only
        // rescaled) when a score exceeds it by more than 8 in log2 units, so
        // every p = exp2((s - m_run) * scale * log2 e) stays <= 2^8.  The final
        // O / l is the same softmax whichever reference max was used.
        if (__ballot(mx > m_run + rescale_thr) != 0) {  // wave-uniform branch
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
        }
        const float mb = m_run * scale_log2;
        float rs0 = 0.f, rs1 = 0.f;
        float p12[2] = {0.f, 0.f};  // pair 12 until it joins the row sums (blocked)
        uint32_t pw[4][4];  // bf16 pairs of P: B operands of the 4 PV steps
        float mxn = -INFINITY;

        // ---- software-pipelined slots.  Slots 0..15: S_{n+1} = K_{n+1} Q^T
        // (s = u/2, tile mt = u%2).  Slots 16..31: O^T += V^T_n P^T_n (step
        // cc = (u-16)/4, d tile dt = (u-16)%4).  The 16 pairs of exponentials of sub-tile n are spread over the
        // slots so that every P group is ready before its PV step, and the row
        // max of S_{n+1} is taken in the last slots, after its MFMAs finished.
        // LDS operands are read in groups of 4, one group ahead of the slots
        // that consume them, so any wait for LDS data lands on reads issued
        // four slots (about 130 cycles) earlier.
        auto read_v = [&](int w) {  // operand of PV slot w
          if constexpr (RASTER) {
            // keys 16*(w/4) + 8*half + 0..7 of d column
            // 64*(l32/16) + 16*(w%4) + l32%16
            const char* bp = reinterpret_cast<const char*>(vn) + vtr +
                             (16 * (w / 4)) * (kRasterVRow * 16) + 32 * (w % 4);
            const v4i16 lo = lds_read_tr16(bp);
            const v4i16 hi = lds_read_tr16(bp + 4 * (kRasterVRow * 16));
            opv[w % 8] = __builtin_bit_cast(ev8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            opv[w % 8] = as_ev8(vn[vread + (w % 4) * 32 * kVRow + 2 * (w / 4)]);
          }
        };
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) nxt[mt][j] = 0.f;
        slot_fence();
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          // this sub-tile's copies, K in the QK^T half and V in the PV half
          // (raster kernel: in slots 2, 6, 10 and 18, 22, 26, which measured
          // 0.4-1% faster there and made no difference to the blocked one)
          if constexpr (kSlotCopies) {
#pragma unroll
            for (int x = 0; x < kMaxK; ++x)
              if (u == (RASTER ? 2 + 4 * x : 1 + (x * 16) / kMaxK)) copy_k(sk, ko[x], x, kw);
#pragma unroll
            for (int x = 0; x < kMaxV; ++x)
              if (u == (RASTER ? 18 + 4 * x : 17 + (x * 16) / kMaxV)) copy_v(sv, vo[x], x, vw);
          }
          if (u < 16) {
            const int s = u / 2, mt = u % 2;
            if (u % 4 == 0) {
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                if (u + 4 < 16) read_k(u + 4 + x);
                else read_v(x);  // first V operands of the PV slots
              }
            }
            nxt[mt] = mfma_32x32x16<F16>(opk[u % 8], qf[s], nxt[mt]);
          } else {
            const int w = u - 16, cc = w / 4, dt = w % 4;
            if (w % 4 == 0 && w + 4 < 16) {
#pragma unroll
              for (int x = 0; x < 4; ++x) read_v(w + 4 + x);
            }
            const ev8 pb = __builtin_bit_cast(
                ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2], pw[cc][3]));
            oacc[dt] = mfma_32x32x16<F16>(opv[w % 8], pb, oacc[dt]);
          }
          // exponential pair e (keys 2e, 2e+1 of this lane's 32).  Blocked
          // kernel: pairs 0..11 in the odd slots 1..23, pair 12 in slot 22
          // and pairs 13..15 in slots 25..27, away from the slots that wait
          // for an LDS operand group (0, 4, ..., 24); pair 12 joins the row
          // sums in slot 25, so the pairs are summed in ascending order as
          // in the raster kernel.  Raster kernel (whose transposing V reads
          // measured better so): pairs 0..11 in the even slots 0..22, pairs
          // 12..15 in slots 24..27.
          int e;
          if constexpr (RASTER)
            e = (u < 24) ? ((u % 2 == 0) ? u / 2 : -1) : ((u < 28) ? u - 12 : -1);
          else
            e = (u < 24 && u % 2 == 1) ? u / 2 : u == 22 ? 12 : (u >= 25 && u < 28) ? u - 12 : -1;
          if (!RASTER && u == 25) {
            rs0 += p12[0];
            rs1 += p12[1];
          }
          if (e >= 0) {
            const int cc = e / 4, t = 2 * (e % 4);
            float p0 = __builtin_amdgcn_exp2f(fmaf(cur[cc / 2][8 * (cc % 2) + t], scale_log2, -mb));
            float p1 = __builtin_amdgcn_exp2f(fmaf(cur[cc / 2][8 * (cc % 2) + t + 1], scale_log2, -mb));
            if (!RASTER && e == 12) {
              p12[0] = p0;
              p12[1] = p1;
            } else {
              rs0 += p0;
              rs1 += p1;
            }
            pw[cc][t / 2] = pack2<F16>(p0, p1);
            pin(rs0);
            pin(rs1);
            pin(pw[cc][t / 2]);
          }
          // row max of S_{n+1}, 4 accumulator registers per slot in slots 24..31
          if (u >= 24) {
            const int mt = (u - 24) / 4, j0 = ((u - 24) % 4) * 4;
            mxn = fmaxf(fmaxf(mxn, nxt[mt][j0]), nxt[mt][j0 + 1]);
            mxn = fmaxf(fmaxf(mxn, nxt[mt][j0 + 2]), nxt[mt][j0 + 3]);
            pin(mxn);
          }
          slot_fence();
        }
        l_run += rs0 + rs1;
        mx_pre = mxn;
      } else if constexpr (kSlotCopies) {
#pragma unroll
        for (int x = 0; x < kMaxK; ++x) copy_k(sk, ko[x], x, kw);
#pragma unroll
        for (int x = 0; x < kMaxV; ++x) copy_v(sv, vo[x], x, vw);
      }
      wait_loads();
      __syncthreads();
      ++n;
      d0 = d1;
      d1 = d2;
      d2 = __builtin_amdgcn_readfirstlane(d3);
    };

    while (true) {
      step(sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
      if (n >= T) break;
      step(sb, sa, kbuf0, kbuf1, vbuf1, vbuf0);
      if (n >= T) break;
    }
  }
  };
  // The 8-wave kernel: one instantiation of the alternating pipeline per
  // wave role (group, key-half or full wave, with or without query rows);
  // a wave's role is fixed for the row, so each keeps its own registers.
  auto pp_rows = [&](auto hv, auto gbt, auto comp) __attribute__((always_inline)) {
    for (int e0 = 0; e0 < len; e0 += kList) {
      const int T = build_list(e0);
      if (T == 0) continue;
      // every global load so far (the Q fragments, the row's column
      // indices) has landed; said in a form the compiler tracks, since it
      // does not count the pipeline's copies and would otherwise wait for
      // them where Q is first used
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
      // descriptor of sub-tile n; past the end it repeats the last one, whose
      // copies then land in buffers that are not read again
      auto desc_at = [&](int n) __attribute__((always_inline)) { return tlist[min(n, T - 1)]; };
      pp_pipeline(hv, gbt, comp, T, desc_at);
    }
  };
  if constexpr (kPP) {
    using F = std::false_type;
    using Tr = std::true_type;
    if (wave < 4) {
      if (!active) pp_rows(F(), F(), F());
      else if (split4) pp_rows(Tr(), F(), Tr());
      else pp_rows(F(), F(), Tr());
    } else {
      if (!active) pp_rows(F(), Tr(), F());
      else if (khalf >= 0) pp_rows(Tr(), Tr(), Tr());
      else pp_rows(F(), Tr(), Tr());
    }
  } else if constexpr (kAllSplit) {
    passes(std::true_type());
  } else {
    if (khalf >= 0) passes(std::true_type());
    else passes(std::false_type());
  }

  // ---- key-half pairs: the second wave of a pair hands its (m, l, O^T) to
  // the first through LDS, which merges them:
  // m = max(m_a, m_b), O = O_a 2^((m_a - m)c) + O_b 2^((m_b - m)c), l likewise.
  // Alternating pipeline: wave 4+x's in V ring slot x (x < 3) or K ring slot
  // 3; 8 waves otherwise: wave 6's in vbuf1, wave 7's in tlist + escan; 4
  // waves: wave 2's in vbuf1, wave 3's in vbuf0 (none of which the epilogue's
  // staging of the rows' owners uses).  The second waves of the pairs own
  // padding rows (zeroed): waves 6, 7 of a 5-6 group block, waves 4..7 of a
  // block of at most 4 groups; waves 2, 3 of a 64-token block own no rows.
  const bool own_pad = (split || split4) && khalf == 1;
  const bool owns_rows = wave * 32 < kVol;
  if (split || split4) {
    float* part;
    if constexpr (kPP) {
      const int pidx = khalf == 1 ? wave - 4 : (split4 ? wave : wave - 2);
      part = reinterpret_cast<float*>(pidx < 3 ? vring + pidx * kVUnits : kring + 3 * kKUnits);
    } else {
      part = (wave & 1) == 0 ? reinterpret_cast<float*>(vbuf1)
                             : (kAllSplit ? reinterpret_cast<float*>(vbuf0)
                                          : reinterpret_cast<float*>(tlist));
    }
    float* const part_ml = kPP || (wave & 1) == 0 || kAllSplit ? part + 64 * 64
                                                               : reinterpret_cast<float*>(escan);
    static_assert(4 * (64 * 64 + 128) <= 16 * kKUnits, "a merge buffer fits a K tile buffer");
    if (own_pad && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) part[(dt * 16 + j) * 64 + lane] = oacc[dt][j];
      part_ml[lane] = m_run;
      part_ml[64 + lane] = l_run;
    }
    __syncthreads();
    if (khalf == 0 && active) {
      const float mb = part_ml[lane], lb = part_ml[64 + lane];
      const float m_new = fmaxf(m_run, mb);
      const float wa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      const float wb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mb - m_new) * scale_log2);
      m_run = m_new;
      l_run = l_run * wa + lb * wb;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          oacc[dt][j] = oacc[dt][j] * wa + part[(dt * 16 + j) * 64 + lane] * wb;
    }
  }

  // ---- tail split: both halves of a split row leave their unnormalised
  // (O^T, m, l) in the slot's part of the workspace (every wave holding rows
  // stores its registers lane by lane); the half whose count comes second
  // reads the other's and merges, with the first half as a and the second
  // as b whichever merges: m = max(m_a, m_b), O = O_a w_a + O_b w_b,
  // l = l_a w_a + l_b w_b, w = 2^((m_x - m) c), each product and sum rounded
  // on its own, so the row's bits do not depend on which half finishes last.
  // The halves may run on different XCDs, whose L2 caches are not coherent
  // with each other: the partials are written and read with device-coherent
  // accesses (relaxed atomic stores and loads at agent scope, which go past
  // the non-coherent L2), the stores drained before the count.  A release or
  // acquire fence would instead write back or invalidate the whole L2 of the
  // XCD, under every other workgroup running there.
  if (part >= 0) {
    const int slot = part >> 1, hf = part & 1;
    const bool holds = active && !own_pad;
    float* const mine = ts.part + (size_t(2 * slot + hf) * NW + wave) * kSplitHalfFloatsPerWave;
    auto put = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto get = [](const float* p) {
      return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (holds) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) put(mine + (dt * 16 + j) * 64 + lane, oacc[dt][j]);
      put(mine + 64 * 64 + lane, m_run);
      put(mine + 65 * 64 + lane, l_run);
    }
    // every store of this wave has reached the coherent level before any
    // wave of the workgroup counts the half as done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ unsigned int done_sh;
    if (tid == 0) done_sh = atomicAdd(&ts.flags[slot], 1u);
    __syncthreads();
    if (done_sh == 0) return;  // the other half merges (workgroup-uniform)
    if (tid == 0) ts.rows[slot] = int32_t(r);
    const float* const other =
        ts.part + (size_t(2 * slot + (1 - hf)) * NW + wave) * kSplitHalfFloatsPerWave;
    if (holds) {
      const float m_o = get(other + 64 * 64 + lane);
      const float l_o = get(other + 65 * 64 + lane);
      const float ma = hf == 0 ? m_run : m_o, mb = hf == 0 ? m_o : m_run;
      const float la = hf == 0 ? l_run : l_o, lb = hf == 0 ? l_o : l_run;
      const float m_new = fmaxf(ma, mb);
      const float wa = ma == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ma - m_new) * scale_log2);
      const float wb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mb - m_new) * scale_log2);
      m_run = m_new;
      l_run = __fadd_rn(__fmul_rn(la, wa), __fmul_rn(lb, wb));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float ov = get(other + (dt * 16 + j) * 64 + lane);
          const float oa = hf == 0 ? oacc[dt][j] : ov, ob = hf == 0 ? ov : oacc[dt][j];
          oacc[dt][j] = __fadd_rn(__fmul_rn(oa, wa), __fmul_rn(ob, wb));
        }
    }
  }

  // ---- epilogue: combine the two lane halves' partial sums, normalise, and
  // store O through LDS so that every global store is a full 256-byte row.
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool row_valid = active && !own_pad && qrow < cq;
  const float inv = (row_valid && l_run > 0.f) ? 1.f / l_run : 0.f;
  // staging area of 32 rows x 272 B per wave: two waves per buffer
  uint4* const sbase = kPP ? kring + (wave / 2) * kKUnits
                            : (wave < 2 ? kbuf0 : (wave < 4 ? kbuf1 : (wave < 6 ? vbuf0 : vbuf1)));
  uint4* const srows = sbase + (wave % 2) * 32 * kORow;
  uint2* const ostage = reinterpret_cast<uint2*>(srows);
#pragma unroll
  for (int dt = 0; dt < 4 && !own_pad; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // registers 4jj..4jj+3 hold O^T rows m = 8jj + 4*half + 0..3, i.e.
      // d = 32dt + m (blocked) or 64*(m/16) + 16dt + m%16 (raster)
      const int d0 = RASTER ? 64 * (jj / 2) + 16 * dt + 8 * (jj % 2) + 4 * half
                            : dt * 32 + 8 * jj + 4 * half;
      const uint2 w = make_uint2(
          pack2<F16>(oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv),
          pack2<F16>(oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv));
      ostage[l32 * (kORow * 2) + d0 / 4] = w;
    }
  // the staging area of wave w is only touched by wave w
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (RASTER) {
    // rows go to their raster tokens; pad rows are dropped.  With a gate the
    // row is O + gate * oc[block i] in fp32, rounded once (as the gated scatter).
    const int unit = lane & 15;
    float c[8];
    if (gate != nullptr) {
      const float4* cp = reinterpret_cast<const float4*>(oc + (bh * g.nb + i) * kHeadDim + unit * 8);
      const float4 c0 = cp[0], c1 = cp[1];
      c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
      c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    }
    const int64_t obase = head0 + origin_i * rs + unit;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int rr = p * 4 + lane / 16;
      const int slot = wave * 32 + rr;
      if (slot < cq && !own_pad) {
        const int64_t at = obase + soff[cls_i * kVol + slot];
        uint4 val = srows[rr * kORow + unit];
        if (gate != nullptr) {
          const uint4 gv = gate[at];
          const uint32_t ow[4] = {val.x, val.y, val.z, val.w};
          const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack2<F16>(fmaf(elem_to_f32<F16>(gw[e] & 0xffffu), c[2 * e],
                                   elem_to_f32<F16>(ow[e] & 0xffffu)),
                              fmaf(elem_to_f32<F16>(gw[e] >> 16), c[2 * e + 1],
                                   elem_to_f32<F16>(ow[e] >> 16)));
          val = make_uint4(w[0], w[1], w[2], w[3]);
        }
        o[at] = val;
      }
    }
  } else if (owns_rows) {
    uint4* const odst = o + (qk_row0 + wave * 32) * 16;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int rr = p * 4 + lane / 16;
      odst[rr * 16 + (lane & 15)] =
          own_pad ? make_uint4(0u, 0u, 0u, 0u) : srows[rr * kORow + (lane & 15)];
    }
  }
  if (lse != nullptr && half == 0 && owns_rows) {
    lse[qk_row0 + (own_pad ? wave * 32 + l32 : qrow)] =
        (row_valid && l_run > 0.f) ? m_run * scale + __logf(l_run) : -INFINITY;
  }
}

// Rows of each of the 8 queue ranges of the balanced launch in claim order,
// for block maps whose rows differ in length.  First the range's long rows
// (entry count >= 4x the range's mean), in ascending row order, so that none
// of them starts late; then the other rows head by head (a head is a run of
// nb consecutive rows), within a head by entry count, largest first, equal
// counts in ascending row order.  The workgroups running at once on an XCD
// then hold rows of one head with about the same number of key blocks, and as
// every row's column list is streamed in ascending order they move through
// the head's key blocks in step and share them in the XCD's L2: the key and
// value blocks of one head of a random map are several times the L2, and
// rows at different points of their lists would each miss.
// order[start .. start + count) of range x is a permutation of the range's
// rows; claim_row hands positions out in that order.  Range x has G
// workgroups (G = gridDim.x / 8, at most 32): workgroup g sorts the heads g,
// g + G, g + 2G, ... that the range touches, in that order, counting the rows
// between them as it goes (so each reads the range's lengths about once), and
// workgroup 0 also places the long rows.  Offsets are sanitised as the
// attention kernel sanitises them.
__global__ __launch_bounds__(1024) void order_rows_kernel(const int32_t* __restrict__ row_ptr,
                                                          int64_t nnz, int64_t nrows, int nb,
                                                          int32_t* __restrict__ order) {
  constexpr int kBins = 2048;   // entry counts >= kBins - 1 share the first bin
  constexpr int kCache = 4096;  // row lengths kept in LDS when the range has at most this many rows
  __shared__ long long wsum[16];
  __shared__ int lens_sh[kCache];
  __shared__ int wcnt[16];
  __shared__ int bin_at[kBins];  // count, then first position, of each bin of a head
  __shared__ __align__(16) int keys[1024];
  const uint32_t n = uint32_t(nrows), per = n / 8, rem = n % 8, x = blockIdx.x % 8,
                 seg = blockIdx.x / 8, nseg = gridDim.x / 8;
  const uint32_t start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  const uint32_t count = per + (x < rem ? 1u : 0u);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  auto len_of = [&](uint32_t r) -> int64_t {
    const int64_t beg = min(max(int64_t(row_ptr[r]), int64_t(0)), nnz);
    const int64_t end = min(max(int64_t(row_ptr[r + 1]), beg), nnz);
    return end - beg;
  };
  // the lengths are read from global memory once and kept in LDS (the passes
  // below read each several times); a longer range reads them each time
  const bool cached = count <= uint32_t(kCache);
  auto len = [&](uint32_t r) -> int64_t { return cached ? lens_sh[r - start] : len_of(r); };
  // total entries of the range
  long long part = 0;
  for (uint32_t t = tid; t < count; t += 1024) {
    const int64_t l = len_of(start + t);
    if (cached) lens_sh[t] = int(min(l, int64_t(0x7fffffff)));
    part += l;
  }
  for (int d = 32; d > 0; d /= 2) part += __shfl_xor(part, d);
  if (lane == 0) wsum[wave] = part;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < 16; ++w) total += wsum[w];
  // long row: len*count >= 4*total (integer arithmetic)
  auto is_long = [&](int64_t l) { return (long long)l * (long long)count >= 4 * total; };
  // bin of a row that is not long: 0 for the largest counts
  auto bin_of = [&](int64_t l) { return kBins - 1 - int(min(l, int64_t(kBins - 1))); };

  if (count == 0 || nb <= 0) return;
  const uint32_t last = start + count;
  const uint32_t head0 = start - start % uint32_t(nb);  // first row of the range's first head
  if (uint64_t(head0) + uint64_t(seg) * uint32_t(nb) >= last) return;  // workgroup-uniform

  // the long rows, ascending (ballot compaction, 1024 rows at a time), placed
  // by workgroup 0; every workgroup counts them
  uint32_t nlong = 0;
  for (uint32_t chunk = 0; chunk < count; chunk += 1024) {
    const uint32_t t = chunk + tid;
    const bool flag = t < count && is_long(len(start + t));
    const unsigned long long b = __ballot(flag);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    __syncthreads();  // wcnt of the previous chunk has been read by everyone
    if (lane == 0) wcnt[wave] = __popcll(b);
    __syncthreads();
    int woff = 0, ctot = 0;
    for (int w = 0; w < 16; ++w) {
      woff += w < wave ? wcnt[w] : 0;
      ctot += wcnt[w];
    }
    if (flag && seg == 0) order[start + nlong + woff + before] = int32_t(start + t);
    nlong += ctot;
  }

  // this workgroup's heads, ascending; `prior` counts the rows that are not
  // long in [start, scanned)
  uint32_t scanned = start, prior = 0;
  for (uint32_t hs = seg;; hs += nseg) {
    const uint64_t h0 = uint64_t(head0) + uint64_t(hs) * uint32_t(nb);  // no wrap-around
    if (h0 >= last) break;  // workgroup-uniform
    const uint32_t s0 = max(uint32_t(h0), start);
    const uint32_t s1 = uint32_t(min(h0 + uint32_t(nb), uint64_t(last)));
    int c = 0;
    for (uint32_t t = scanned + tid; t < s0; t += 1024) c += is_long(len(t)) ? 0 : 1;
    for (int d = 32; d > 0; d /= 2) c += __shfl_xor(c, d);
    __syncthreads();  // wcnt of the previous pass has been read
    if (lane == 0) wcnt[wave] = c;
    __syncthreads();
    for (int w = 0; w < 16; ++w) prior += uint32_t(wcnt[w]);
    scanned = s0;
    const uint32_t base = nlong + prior;

    // the head's other rows: a counting sort by bin
    for (int b = tid; b < kBins; b += 1024) bin_at[b] = 0;
    __syncthreads();
    for (uint32_t t = s0 + tid; t < s1; t += 1024) {
      const int64_t l = len(t);
      if (!is_long(l)) atomicAdd(&bin_at[bin_of(l)], 1);
    }
    __syncthreads();
    // exclusive scan of the bin counts (two bins per thread)
    const int c0 = bin_at[2 * tid], c1 = bin_at[2 * tid + 1];
    int incl = c0 + c1;
    for (int d = 1; d < 64; d *= 2) {
      const int up = __shfl_up(incl, d);
      if (lane >= d) incl += up;
    }
    __syncthreads();  // wcnt of the counts above has been read
    if (lane == 63) wcnt[wave] = incl;
    __syncthreads();
    int woff = 0;
    for (int w = 0; w < 16; ++w) woff += w < wave ? wcnt[w] : 0;
    const int excl = woff + incl - (c0 + c1);
    bin_at[2 * tid] = excl;
    bin_at[2 * tid + 1] = excl + c0;
    __syncthreads();
    // place the head's rows 1024 at a time: a row's position is its bin's
    // next free position plus the rows of the same bin before it in the chunk
    for (uint32_t chunk = s0; chunk < s1; chunk += 1024) {
      const uint32_t t = chunk + tid;
      int key = -1;
      if (t < s1) {
        const int64_t l = len(t);
        if (!is_long(l)) key = bin_of(l);
      }
      keys[tid] = key;
      __syncthreads();
      int same = 0;
      if (key >= 0) {
        const int4* k4 = reinterpret_cast<const int4*>(keys);
        const int n4 = tid / 4;
        int j = 0;
        for (; j + 8 <= n4; j += 8) {  // eight reads in flight at a time
          int4 kk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) kk[u] = k4[j + u];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            same += (kk[u].x == key) + (kk[u].y == key) + (kk[u].z == key) + (kk[u].w == key);
        }
        for (; j < n4; ++j) {
          const int4 kk = k4[j];
          same += (kk.x == key) + (kk.y == key) + (kk.z == key) + (kk.w == key);
        }
        for (int q = tid & ~3; q < tid; ++q) same += keys[q] == key;
        order[start + base + bin_at[key] + same] = int32_t(t);
      }
      __syncthreads();  // every row of the chunk has read bin_at
      if (key >= 0) atomicAdd(&bin_at[key], 1);
      __syncthreads();
    }
  }
}

template <int NW, int NQ, bool F16, bool RASTER>
hipError_t launch_nw(const VsaGeom& g, const void* q, const void* k, const void* v,
                     const int32_t* row_ptr, const int32_t* col, int uniform_k, int64_t nnz,
                     void* o, float* lse, const void* gate, const float* oc,
                     unsigned int* queues, int32_t* order, TailSplit ts, hipStream_t s) {
  const int64_t rows = int64_t(g.batch) * g.heads * g.nb;
  const float scale = 1.0f / sqrtf(float(g.head_dim));
  const float scale_log2 = scale * 1.4426950408889634f;
  int64_t grid = rows;
  const int32_t* claim_order = nullptr;
  if (queues == nullptr || ts.flags == nullptr) ts.per_queue = 0;
  {
    // rows of the longest queue under the claim rule the kernel will use
    const bool strided = row_ptr == nullptr && g.head_interleave;
    const int64_t qmax =
        strided ? int64_t((g.nb + 7) / 8) * g.batch * g.heads : (rows + 7) / 8;
    if (qmax > kSplitMaxQueueRows) ts.per_queue = 0;
  }
  if (queues != nullptr) {
    // a quarter more workgroups than items (rows, plus one more for each
    // split row), so that each XCD can take up to 1.25 times its share; the
    // counters are cleared first on the same stream
    const int64_t items = rows + split_slots_max(g, ts.per_queue);
    grid = items + std::max<int64_t>(8, items / 4);
    const int nflags = int(split_slots_max(g, ts.per_queue));
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(256), 0, s, queues, ts.flags, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (row_ptr != nullptr && order != nullptr) {
      // workgroups per queue range: the heads a range can touch (its rows,
      // plus one for a range that starts inside a head), at most 32
      const int64_t per_max = (rows + 7) / 8;
      const int64_t segs = std::min<int64_t>(32, (per_max + g.nb - 1) / g.nb + 1);
      hipLaunchKernelGGL(order_rows_kernel, dim3(unsigned(8 * segs)), dim3(1024), 0, s, row_ptr,
                         nnz, rows, g.nb, order);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      claim_order = order;
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<NW, NQ, F16, RASTER>), dim3(unsigned(grid)), dim3(NW * 64),
                     0, s, static_cast<const uint4*>(q), static_cast<const uint4*>(k),
                     static_cast<const uint4*>(v), row_ptr, col, uniform_k, nnz,
                     static_cast<uint4*>(o), lse, static_cast<const uint4*>(gate), oc, queues,
                     claim_order, g, scale_log2, scale, ts);
  return hipGetLastError();
}

template <bool RASTER>
hipError_t launch_any(const VsaGeom& g, const void* q, const void* k, const void* v,
                      const int32_t* row_ptr, const int32_t* col, int uniform_k, int64_t nnz,
                      void* o, float* lse, const void* gate, const float* oc,
                      unsigned int* queues, int32_t* order, const TailSplit& ts,
                      hipStream_t s) {
  auto launch = [&](auto nw, auto nq) {
    constexpr int NW = decltype(nw)::value, NQ = decltype(nq)::value;
    return g.dtype == VSA_DTYPE_FP16
               ? launch_nw<NW, NQ, true, RASTER>(g, q, k, v, row_ptr, col, uniform_k, nnz, o,
                                                 lse, gate, oc, queues, order, ts, s)
               : launch_nw<NW, NQ, false, RASTER>(g, q, k, v, row_ptr, col, uniform_k, nnz, o,
                                                  lse, gate, oc, queues, order, ts, s);
  };
  using std::integral_constant;
  switch (g.vol / 32) {
    case 2: return launch(integral_constant<int, 4>(), integral_constant<int, 2>());
    case 4: return launch(integral_constant<int, 4>(), integral_constant<int, 4>());
    case 6: return launch(integral_constant<int, 6>(), integral_constant<int, 6>());
    case 8: return launch(integral_constant<int, 8>(), integral_constant<int, 8>());
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  // Each device holds its own copy of `scratch` at its own address: look it
  // up once per device, with that device current, and keep it.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_attn_fwd(const VsaGeom& g, const void* q, const void* k, const void* vt,
                           const int32_t* row_ptr, const int32_t* col, int uniform_k,
                           int64_t nnz, void* o, float* lse, unsigned int* queues,
                           int32_t* order, const TailSplit& ts, hipStream_t s) {
  return launch_any<false>(g, q, k, vt, row_ptr, col, uniform_k, nnz, o, lse, nullptr, nullptr,
                           queues, order, ts, s);
}

hipError_t launch_attn_fwd_raster(const VsaGeom& g, const void* q, const void* k, const void* v,
                                  const int32_t* row_ptr, const int32_t* col, int uniform_k,
                                  int64_t nnz, void* o, float* lse, const void* gate,
                                  const float* oc, unsigned int* queues, int32_t* order,
                                  const TailSplit& ts, hipStream_t s) {
  return launch_any<true>(g, q, k, v, row_ptr, col, uniform_k, nnz, o, lse, gate, oc, queues,
                          order, ts, s);
}

}  // namespace vsa
