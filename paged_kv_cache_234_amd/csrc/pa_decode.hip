// Paged decode attention for gfx950: persistent wave streaming.
//
// Operation: grouped-query softmax(scale * q K^T) V for one query token per
// sequence, over a paged cache (infer-lab: technique table, PagedAttention
// row; layout section, GQA; tiled online-softmax attention; llm-infer, "What
// It Does": a paged KV cache with block tables; the tiling follows the
// FlashAttention-2 reference llm-infer cites).  With partition_size > 0 the
// context is cut into fixed partitions whose softmax partials (m, l, o) are
// merged by pa_decode_splitk_reduce (flash-decoding split-K).
//
// Rows.  The kernel walks a list of rows.  Row b < batch is sequence b: its
// 16 MFMA columns are the G query heads of one KV head (G <= 16, so every
// K/V byte is read once per sequence).  The cascade entry point adds one row
// per prefix group (sequences whose first tokens sit in the same physical
// blocks, infer-lab RadixAttention row, llm-infer prefix caching): its
// columns are (member, query head) pairs, 16 / G members at a time, and it
// covers the whole partitions of the shared prefix once for all members.
// The members' own rows then skip those partitions.  A group row has one
// "virtual head" per (KV head, 16-column chunk of members); the chunks of one
// KV head are adjacent, so they read the same blocks back to back.
//
// Work decomposition.  A work item is (row, virtual head, partition).  Tiles
// of TT positions are numbered row-major, then virtual head, then position;
// each workgroup builds the prefix of per-row tile counts in LDS.  With s(g)
// the item start nearest to tile g, range k holds the whole items whose
// first tile lies in [s(T k / NWG), s(T (k+1) / NWG)), which is within half
// an item of an equal share; its NW wavefronts split that run into NW equal
// runs of tiles.  Workgroup k takes range k (plain rows) or the range that
// keeps runs of 8 consecutive ranges on one XCD (group and multi-query rows,
// whose neighbouring items may read the same K/V).  A wavefront
// streams its tiles back to back: the next tile's K/V loads -- across item
// boundaries too -- are in flight while the current tile is multiplied, and a
// finished item writes its partial (or output) straight from registers.
//
// Items cut between wavefronts.  Every item is computed as one online softmax
// over its tiles in order, whichever wavefronts hold them, so an item's result
// does not depend on where the batch around it puts the cuts: a sequence's
// output is the same, bit for bit, alone or in any batch, and a prefix
// partition read for a group row equals the one a member's own row reads
// (infer-lab, invariants: batched decode equals sequential decode, and
// prefix-cached equals uncached).  A wavefront runs its range in the order
// Y, M, X: Y = the first tiles of the item cut at its end, M = its whole
// items, X = the last tiles of the item cut at its start.  After Y it parks
// its running softmax state in LDS; the next wavefront takes that state when
// it reaches its X, last, and continues the same softmax from it.  The state
// is handed on, never merged, so the arithmetic equals one wavefront's.
#include <algorithm>
#include <type_traits>

#include "pa_internal.hpp"
#include "pa_tiles.hpp"
#include "pa_write.hpp"

namespace pa {

constexpr int kMaxDecodeRows = 4096;
constexpr int kStageRows = 34;          // split-K partial rows a plain wavefront collects in LDS (the most that fit)
constexpr int kMaxMultiQuery = 64;     // query tokens per sequence in pa_decode_multi

// Launch plan.  The decode prologue (row table, tile prefix, workgroup and
// wavefront ranges, the first tile's block ids) depends only on the context
// lengths, the block tables and the launch shape, which every layer of a
// decode step shares.  A plan holds it as int32 words:
//   [0, 16)             header (kPlan* fields below)
//   [16, 16 + R)        context length per row (cut as the prologue cuts it)
//   [16 + R, 16 + 2R)   the row's aux word (plain rows: tiles per KV head)
//   [16 + 2R, 17 + 3R)  exclusive prefix of tiles (R + 1 entries)
// for R rows (the sequences, then any prefix groups).
//   then, 16-aligned, 32 words per wavefront (grid x 4): first and end tile,
//   its workgroup's first and end tile, the rows of its first and last tile,
//   the block ids of its first tile (4 words) and of its second (4 words),
//   the number of new tokens it appends (-1: not listed) and, from word 16,
//   up to kPlanMaxAppends (row * num_kv_heads + head, slot) pairs.
enum { kRun = 0, kMakePlan = 1, kUsePlan = 2 };
constexpr int kPlanMagic = 0x50414450;
enum {
    kPlanMagicW, kPlanBatch, kPlanKvHeads, kPlanPS, kPlanMaxPart, kPlanTT, kPlanGrid, kPlanNW,
    kPlanMaxBlocks, kPlanSplit, kPlanTiles, kPlanHeadDim, kPlanRows, kPlanRowKind, kPlanAppends,
    kPlanHeader = 16
};
constexpr int kPlanWave = 32;
constexpr int kPlanMaxAppends = 8;     // tokens a wavefront's words can list
__host__ __device__ constexpr long plan_waves_offset(int batch) {
    return ((long)kPlanHeader + 3L * batch + 1 + 15) / 16 * 16;
}

struct DecodeArgs {
    void* out;
    const void* q;
    const char* k_cache;
    const char* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* part_max;
    float* part_sum;
    float* part_out;
    // prefix groups (cascade): members of group j are
    // group_seqs[group_start[j] .. group_start[j+1]), sharing their first
    // group_prefix_lens[j] positions
    const int32_t* group_start;
    const int32_t* group_seqs;
    const int32_t* group_prefix_lens;
    int num_groups;
    // multi-query rows: sequence b's query tokens are rows
    // query_start_loc[b] .. query_start_loc[b+1]-1 of q and of the partials,
    // at positions L_b - q_len_b .. L_b - 1 (causal among themselves)
    const int32_t* query_start_loc;
    // fused append (plain decode, cascade): sequence b's newest token, at
    // position L_b - 1, goes to slot new_slots[b] (-1: already in the pool)
    const void* k_new;
    const void* v_new;
    const int32_t* new_slots;
    char* k_cache_w;
    char* v_cache_w;
    // launch plan (plain decode): written by pa_decode_plan's launch, read
    // in place of the prologue by later launches over the same batch
    const int32_t* plan;
    int32_t* plan_out;
    int max_blocks_per_seq;
    int batch;
    int num_heads;
    int num_kv_heads;
    int group;             // G
    int partition_size;    // tokens per item (split), or the whole table row (single pass)
    int max_partitions;    // slots per (sequence, query head) in the partial buffers
    int split;             // write partials instead of out
    float scale_log2;      // scale * log2(e)
};

template <int KIND> struct QType { using T = uint16_t; };
template <> struct QType<kF32> { using T = float; };

// Running online-softmax state of an item cut at the end of a wavefront's
// range, parked in LDS for the wavefront that continues the item.
template <int NVT, int NC> struct SegSlot {
    f32x4 o[NC][NVT][kWave];
    float m[NC][kWave], mr[NC][kWave], l[NC][kWave];
};

// Group and multi-query rows balance cost, not tiles, in the ranges a plan
// records: an item costs its tiles plus kWideItemCost (its Q load, its
// partial write and the cursor's turn), so many short items weigh like the
// long ones they stand beside.
constexpr int kWideItemCost = 1;
// A plan whose launches append also charges kAppendCost to the last item of
// each virtual head of a row with a token to append: the wavefront that
// holds it waits for the token's rows before its second tile's loads go out,
// so it takes a little less other work.
constexpr int kAppendCost = 1;

// NC: 16-column query tiles per wavefront.  Sequence rows use one (their
// columns are one KV head's G <= 16 query heads); group and multi-query rows
// give each virtual head NC * 16 columns, so one K/V tile feeds up to
// NC * 16 / G members or query positions.
// PLAIN: sequence rows only (pa_decode); the group and multi-query row code
// is compiled out.
// STAGE: the plain kernel's split-K rows collected in LDS (long ranges only)
template <int KIND, int D, int NW, int NC, bool PLAIN, int MODE, bool CI = false, bool STAGE = false>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(waves_per_simd(KIND, D))))
void decode_kernel(DecodeArgs a) {
    static_assert(!STAGE || (PLAIN && D == 128 && MODE != kMakePlan), "staging: plain rows, head size 128");
    // which rows a plan describes: plain sequences, cascade or multi-query
    const int row_kind = PLAIN ? 0 : (a.query_start_loc != nullptr ? 2 : 1);
    using Ops = TileOps<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int TT = Ops::TT, TB = Ops::TB, NVT = Ops::NVT, ELEM = Ops::ELEM;
    constexpr int NT = NW * kWave;

    // per row: context length; aux = leading partitions covered by the
    // row's prefix group (sequence rows) or (first member index << 16 |
    // members) (group rows); exclusive prefix of tiles
    __shared__ int s_len[kMaxDecodeRows];
    __shared__ int s_aux[kMaxDecodeRows];
    __shared__ int s_tpre[kMaxDecodeRows + 1];
    __shared__ int s_wsum[NW];
    // a plan for group or multi-query rows balances cost (kWideItemCost);
    // exclusive prefix of that cost per row
    constexpr bool kCost = !PLAIN && MODE == kMakePlan;
    constexpr int kItemCost = kCost ? kWideItemCost : 0;
    __shared__ int s_cpre[kCost ? kMaxDecodeRows + 1 : 1];
    __shared__ int s_csum[NW];
    __shared__ int s_wstart[NW + 1];             // the wavefronts' first tiles, then the end
    __shared__ SegSlot<NVT, NC> s_seg[NW];       // state of the item cut at a wave's end
    __shared__ int s_ready[NW];                  // s_seg[w] holds it

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int B = a.batch;
    const int R = PLAIN ? B : B + a.num_groups;
    const int PS = a.partition_size;
    const int tpi = (PS + TT - 1) / TT;                  // tiles of a full item
    const int Hkv = a.num_kv_heads;
    const int mpc = 16 / a.group;                        // members / query positions per 16 columns
    const int mpv = mpc * NC;                            // ... per virtual head
    const bool multi = !PLAIN && a.query_start_loc != nullptr;

    // what the prologue settles: total tiles, this workgroup's and this
    // wavefront's tile ranges, the rows of the wavefront's first and last tile
    int T = 0, wg_a = 0, wg_e = 0, g0 = 0, g1 = 0, rg0 = 0, rg1 = 0;
    int plan_ids[2][Ops::TB];                    // block ids of the first two tiles (from a plan)
    int plan_apps = -1;                          // tokens this wavefront appends (a plan's list)
    int plan_app_rh[kPlanMaxAppends], plan_app_slot[kPlanMaxAppends];
    bool plan_ok = true;
    if constexpr (MODE == kUsePlan) {
        // header and this wavefront's words: scalar loads; the row table
        // goes to LDS.  A plan made for other arguments leaves no work.
        const int32_t* pl = a.plan;
        const int eff_ps = PS, eff_mp = a.max_partitions;
        plan_ok = load_invariant(pl + kPlanMagicW) == kPlanMagic &&
                  load_invariant(pl + kPlanBatch) == B && load_invariant(pl + kPlanKvHeads) == Hkv &&
                  load_invariant(pl + kPlanRows) == R && load_invariant(pl + kPlanRowKind) == row_kind &&
                  load_invariant(pl + kPlanPS) == eff_ps &&
                  load_invariant(pl + kPlanMaxPart) == eff_mp &&
                  load_invariant(pl + kPlanTT) == TT &&
                  load_invariant(pl + kPlanGrid) == (int)gridDim.x &&
                  load_invariant(pl + kPlanNW) == NW &&
                  load_invariant(pl + kPlanMaxBlocks) == a.max_blocks_per_seq &&
                  load_invariant(pl + kPlanSplit) == a.split &&
                  load_invariant(pl + kPlanHeadDim) == D;
        const int32_t* wv = pl + plan_waves_offset(R) + ((long)blockIdx.x * NW + wave) * kPlanWave;
        T = load_invariant(pl + kPlanTiles);
        g0 = load_invariant(wv + 0);
        g1 = load_invariant(wv + 1);
        wg_a = load_invariant(wv + 2);
        wg_e = load_invariant(wv + 3);
        rg0 = load_invariant(wv + 4);
        rg1 = load_invariant(wv + 5);
#pragma unroll
        for (int j = 0; j < Ops::TB; ++j) {
            plan_ids[0][j] = load_invariant(wv + 6 + j);
            plan_ids[1][j] = load_invariant(wv + 10 + j);
        }
        plan_apps = load_invariant(pl + kPlanAppends) == 1 ? load_invariant(wv + 14) : -1;
#pragma unroll
        for (int i = 0; i < kPlanMaxAppends; ++i) {
            plan_app_rh[i] = load_invariant(wv + 16 + 2 * i);
            plan_app_slot[i] = load_invariant(wv + 17 + 2 * i);
        }
        for (int r = tid; r < R; r += NT) {
            s_len[r] = pl[kPlanHeader + r];
            s_aux[r] = pl[kPlanHeader + R + r];
            s_tpre[r] = pl[kPlanHeader + 2 * R + r];
        }
        if (tid == 0) s_tpre[R] = pl[kPlanHeader + 3 * R];
        if (!plan_ok) g0 = g1 = wg_a = wg_e = 0;
    } else {
    // ---- row table in LDS -------------------------------------------------------
    // Group descriptors are read together with the context lengths, and a
    // group's member list in batches of 8 independent loads, so the prologue
    // costs two dependent memory round trips.
    for (int r = tid; r < B; r += NT) {
        // positions past the table row or the partial buffers are never read
        const int L = (int)std::min<long>(a.context_lens[r],
                                          std::min<long>((long)a.max_blocks_per_seq * kBlock,
                                                         (long)a.max_partitions * PS));
        s_len[r] = L;
        s_aux[r] = 0;
        if (multi) {            // (first query row << 8) | queries (<= L, < 256)
            const int q0 = a.query_start_loc[r];
            const int nq = max(0, min(min(a.query_start_loc[r + 1] - q0, L), 255));
            s_aux[r] = (q0 << 8) | nq;
        }
    }
    if (!PLAIN && a.num_groups > 0) {
        constexpr int kBatch = 8;
        for (int j = tid; j < a.num_groups; j += NT) {
            const int first = min(max(a.group_start[j], 0), 0x7FFF);
            const int members = max(0, min(a.group_start[j + 1] - first, 0xFFFF));
            // whole shared partitions, clamped to the partial buffer and the table row
            int full = max(0, a.group_prefix_lens[j]) / PS;
            full = min(full, min(a.max_partitions, a.max_blocks_per_seq * kBlock / PS));
            s_len[B + j] = members > 0 ? full * PS : 0;
            s_aux[B + j] = (first << 16) | members;
        }
        __syncthreads();                                  // s_len of the sequences
        for (int j = tid; j < a.num_groups; j += NT) {
            const int first = s_aux[B + j] >> 16, members = s_aux[B + j] & 0xFFFF;
            const int full = s_len[B + j] / PS;
            for (int m0 = 0; m0 < members; m0 += kBatch) {
                int sq[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    sq[k] = m0 + k < members ? a.group_seqs[first + m0 + k] : -1;
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (sq[k] >= 0 && sq[k] < B)
                        s_aux[sq[k]] = min(full, (s_len[sq[k]] + PS - 1) / PS);
            }
        }
    }
    }
    __syncthreads();

    auto row_skip = [&](int r) { return (!PLAIN && r < B && !multi) ? s_aux[r] : 0; };
    auto row_heads = [&](int r) {
        if (PLAIN || (r < B && !multi)) return Hkv;
        const int cols = r < B ? (s_aux[r] & 0xFF) : (s_aux[r] & 0xFFFF);
        return Hkv * ((cols + mpv - 1) / mpv);
    };
    auto row_items = [&](int r) {
        const int L = s_len[r];
        if (L <= 0) return 0;
        const int n = a.split ? (L + PS - 1) / PS : 1;
        return max(0, n - row_skip(r));
    };
    // tiles of one (virtual) head of row r
    auto head_tiles_of = [&](int r) {
        const int n = row_items(r);
        if (n == 0) return 0;
        const int last = row_skip(r) + n - 1;
        return (n - 1) * tpi + (s_len[r] - last * PS + TT - 1) / TT;
    };
    // extra cost of the last item of each virtual head of row r (plans whose
    // launches append: sequence rows with a position, multi-query rows with
    // a query token)
    auto append_cost = [&](int r) {
        if (!kCost || a.new_slots == nullptr || r >= B || row_items(r) == 0) return 0;
        return (multi ? (s_aux[r] & 0xFF) > 0 : s_len[r] > 0) ? kAppendCost : 0;
    };
    // plain decode keeps it in s_aux (otherwise unused) once the prefix is built
    auto row_head_tiles = [&](int r) { return PLAIN ? s_aux[r] : head_tiles_of(r); };
    // Tile order within a row.  Sequence and group rows: virtual head (KV
    // head h, member chunk ch: vh = h nch + ch), then item (partition).
    // Multi-query launches (CI): KV head, then item, then chunk, so a row
    // whose query columns take nch > 1 chunks per KV head has the chunks of
    // one partition next to each other: neighbouring wavefronts stream the
    // same K/V tiles at the same time and the second read comes from L2.
    // Every item of a partition but the last has tpi tiles, those of the
    // last rem.  The item of row r holding tile g: its first tile t0, its
    // tiles nti, virtual head vh, item p and tile jj within it.
    auto locate = [&](int g, int r, int& t0, int& nti, int& vh, int& p, int& jj) {
        const int th = row_head_tiles(r);
        const int base = s_tpre[r];
        if constexpr (PLAIN || !CI) {                              // virtual head, then item
            vh = (g - base) / th;
            const int j = g - base - vh * th;
            p = j / tpi;
            t0 = base + vh * th + p * tpi;
            jj = j - p * tpi;
            nti = p + 1 < row_items(r) ? tpi : th - p * tpi;
            return;
        }
        const int nch = row_heads(r) / Hkv;
        const int n = row_items(r);
        const int rem = th - (n - 1) * tpi;
        const int hb = nch * th;                                   // tiles of one KV head
        const int h = (g - base) / hb;
        const int jh = g - base - h * hb;
        const int full = (n - 1) * nch * tpi;                      // tiles of the full items
        int ch;
        if (jh < full) {
            p = jh / (nch * tpi);
            const int k = jh - p * nch * tpi;
            ch = k / tpi;
            jj = k - ch * tpi;
            t0 = base + h * hb + p * nch * tpi + ch * tpi;
            nti = tpi;
        } else {
            p = n - 1;
            const int k = jh - full;
            ch = k / rem;
            jj = k - ch * rem;
            t0 = base + h * hb + full + ch * rem;
            nti = rem;
        }
        vh = h * nch + ch;
    };
    auto item_holding = [&](int g, int r, int& t0, int& nti) {
        int vh, p, jj;
        locate(g, r, t0, nti, vh, p, jj);
    };

    // single pass: sequences with L = 0 have no tile; their rows are zeros
    auto zero_empty_rows = [&]() {
        if (a.split) return;
        const long rows = (long)B * a.num_heads * D;
        for (long r = (long)blockIdx.x * NT + tid; r < rows; r += (long)gridDim.x * NT) {
            if (a.context_lens[r / ((long)a.num_heads * D)] <= 0) {
                if (KIND == kF32) reinterpret_cast<float*>(a.out)[r] = 0.f;
                else reinterpret_cast<uint16_t*>(a.out)[r] = 0;
            }
        }
    };
    // A plan made for other arguments: the launch computes nothing, and every
    // element of the output (or of the partial buffers) it was given becomes
    // NaN, so the mistake cannot pass for a result (RustInfer, "Tensor
    // parallelism": fail instead of silently falling back).
    auto poison_outputs = [&]() {
        // rows of the output / partial buffers: sequences, or multi-query tokens
        const long rows = multi ? (long)max(0, load_invariant(a.query_start_loc + B)) : (long)B;
        const long stride = (long)gridDim.x * NT, start = (long)blockIdx.x * NT + tid;
        if (a.split) {
            const long n = rows * a.num_heads * a.max_partitions;
            for (long i = start; i < n; i += stride) {
                a.part_max[i] = __builtin_nanf("");
                a.part_sum[i] = __builtin_nanf("");
            }
            for (long i = start; i < n * D; i += stride) a.part_out[i] = __builtin_nanf("");
        } else {
            const long n = rows * a.num_heads * D;
            for (long i = start; i < n; i += stride) {
                if (KIND == kF32) reinterpret_cast<float*>(a.out)[i] = __builtin_nanf("");
                else reinterpret_cast<uint16_t*>(a.out)[i] = 0x7FC0;
            }
        }
    };
    if constexpr (MODE == kUsePlan) {
        if (plan_ok) zero_empty_rows();
        else poison_outputs();
    } else {
    // ---- prefix of per-row tile counts (each thread: a run of rows) ---------
    const int per = (R + NT - 1) / NT;
    const int r0 = tid * per;
    auto row_cost = [&](int r) {
        return row_heads(r) * (head_tiles_of(r) + kItemCost * row_items(r) + append_cost(r));
    };
    int local = 0, local_c = 0;
    for (int k = 0; k < per; ++k)
        if (r0 + k < R) {
            const int th = head_tiles_of(r0 + k);
            if (PLAIN) s_aux[r0 + k] = th;
            local += row_heads(r0 + k) * th;
            if (kCost) local_c += row_cost(r0 + k);
        }
    int incl = local, incl_c = local_c;                  // inclusive scans within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(incl, off);
        const int uc = kCost ? __shfl_up(incl_c, off) : 0;
        if (lane >= off) {
            incl += u;
            incl_c += uc;
        }
    }
    if (lane == kWave - 1) {
        s_wsum[wave] = incl;
        s_csum[wave] = incl_c;
    }
    __syncthreads();
    int wbase = 0, total_tiles = 0, cbase = 0, total_cost = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wbase += (w < wave) ? s_wsum[w] : 0;
        total_tiles += s_wsum[w];
        cbase += (w < wave) ? s_csum[w] : 0;
        total_cost += s_csum[w];
    }
    {
        int run = wbase + incl - local, run_c = cbase + incl_c - local_c;
        for (int k = 0; k < per; ++k)
            if (r0 + k < R) {
                s_tpre[r0 + k] = run;
                run += row_heads(r0 + k) * (PLAIN ? s_aux[r0 + k] : head_tiles_of(r0 + k));
                if (kCost) {
                    s_cpre[r0 + k] = run_c;
                    run_c += row_cost(r0 + k);
                }
            }
        if (tid == 0) {
            s_tpre[R] = total_tiles;
            if (kCost) s_cpre[R] = total_cost;
        }
    }
    if constexpr (MODE == kRun) zero_empty_rows();
    __syncthreads();

    // ---- tile ranges ----------------------------------------------------------
    // Tile numbers fit in 32 bits (the prefix lives in an int table); the
    // range arithmetic stays in 32-bit integers, off the 64-bit divide path.
    T = total_tiles;

    // For two tiles ga, gb < T at once (their LDS reads overlap): the row r
    // with tpre[r] <= g < tpre[r+1], i.e. the largest such r, searched 64
    // candidates at a time (two LDS round trips for 4096 rows).  tpre is
    // nondecreasing, so the lanes whose candidate qualifies form a prefix of
    // the wave.
    auto row_of2_in = [&](const int* pre, int ga, int gb, int& ra, int& rb) {
        int loa = 0, spa = R, lob = 0, spb = R;
        while (spa > 1 || spb > 1) {
            const int sta = (spa + kWave - 1) / kWave, stb = (spb + kWave - 1) / kWave;
            const int ia = loa + lane * sta, ib = lob + lane * stb;
            const bool oka = spa > 1 && ia < loa + spa && pre[ia] <= ga;
            const bool okb = spb > 1 && ib < lob + spb && pre[ib] <= gb;
            const int ca = __builtin_popcountll(__builtin_amdgcn_ballot_w64(oka));
            const int cb = __builtin_popcountll(__builtin_amdgcn_ballot_w64(okb));
            if (spa > 1) {
                const int end = loa + spa;
                loa += (ca - 1) * sta;
                spa = min(sta, end - loa);
            }
            if (spb > 1) {
                const int end = lob + spb;
                lob += (cb - 1) * stb;
                spb = min(stb, end - lob);
            }
        }
        ra = loa;
        rb = lob;
    };
    auto row_of2 = [&](int ga, int gb, int& ra, int& rb) { row_of2_in(s_tpre, ga, gb, ra, rb); };
    // the item start nearest to tile g < T in row r (the earlier one on a tie)
    auto nearest_item_start = [&](int g, int r) -> int {
        int before, nti;
        item_holding(g, r, before, nti);
        const int after = before + nti;
        return (g - before <= after - g) ? before : after;
    };
    // X k / NWG, exact: the double product is below 2^53 and a non-integral
    // quotient stays at least 1 / (X k) away from the next integer
    auto share = [&](int x, int k) { return (int)((double)x * k / (double)gridDim.x); };
    // Range k of the wide kernels goes to a block that runs on the same XCD
    // as ranges k - 1 and k + 1 (runs of 8; blocks are dealt round-robin to
    // the XCDs, each with its own L2): a multi-query row's two 32-column
    // chunks of one partition, neighbours in the tile order, then read their
    // K/V through one L2 even when a range boundary falls between them.
    const int kb = PLAIN ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    if constexpr (!kCost) {
        const int sa = share(T, kb), se = share(T, kb + 1);
        if (T > 0) {
            int rsa, rse;
            row_of2(min(sa, T - 1), min(se, T - 1), rsa, rse);
            wg_a = sa >= T ? T : nearest_item_start(sa, rsa);
            wg_e = se >= T ? T : nearest_item_start(se, rse);
        }
        g0 = wg_a + (wg_e - wg_a) * wave / NW;
        g1 = wg_a + (wg_e - wg_a) * (wave + 1) / NW;
    } else {
        // the same on cost: workgroup k takes the items between the item
        // starts nearest to costs C k / NWG and C (k+1) / NWG, and its
        // wavefronts split that run into equal costs (at tile granularity)
        const int C = total_cost;
        const int ci = tpi + kItemCost;                   // cost of a full item
        // the item of row r holding cost c, in the tile order above: its KV
        // head's first tile and cost, the offset o of c in the head, and the
        // item's first tile, first cost and tiles relative to the head
        struct ItemAt {
            int tile0, cost0, o, it_t0, it_c0, nti, ic;
        };
        auto item_at_cost = [&](int c, int r) {
            ItemAt it;
            const int th = head_tiles_of(r), n = row_items(r), ea = append_cost(r);
            const int nch = CI ? row_heads(r) / Hkv : 1;      // (otherwise each virtual head is a unit)
            const int rem = th - (n - 1) * tpi;
            const int chead = nch * (th + kItemCost * n + ea);    // cost of one KV head
            const int h = (c - s_cpre[r]) / chead;
            it.tile0 = s_tpre[r] + h * nch * th;
            it.cost0 = s_cpre[r] + h * chead;
            it.o = c - it.cost0;
            const int full_c = (n - 1) * nch * ci;                // cost of the full items
            if (it.o < full_c) {
                const int k = it.o / ci;
                it.it_c0 = k * ci;
                it.it_t0 = k * tpi;
                it.nti = tpi;
                it.ic = ci;
            } else {
                const int cr = rem + kItemCost + ea;
                const int j = min((it.o - full_c) / cr, nch - 1);
                it.it_c0 = full_c + j * cr;
                it.it_t0 = (n - 1) * nch * tpi + j * rem;
                it.nti = rem;
                it.ic = cr;
            }
            return it;
        };
        auto nearest_item_by_cost = [&](int c, int r, int& tile, int& cost) {
            const ItemAt it = item_at_cost(c, r);
            const int before = it.it_c0, after = it.it_c0 + it.ic;
            const bool take_before = it.o - before <= after - it.o;
            tile = it.tile0 + it.it_t0 + (take_before ? 0 : it.nti);
            cost = it.cost0 + (take_before ? before : after);
        };
        auto tile_at_cost = [&](int c, int r) {           // inside an item, or its successor's start
            const ItemAt it = item_at_cost(c, r);
            return it.tile0 + it.it_t0 + min(it.o - it.it_c0, it.nti);
        };
        int ca = 0, ce = 0;
        const int sa = share(C, kb), se = share(C, kb + 1);
        if (C > 0) {
            int rsa, rse;
            row_of2_in(s_cpre, min(sa, C - 1), min(se, C - 1), rsa, rse);
            if (sa >= C) {
                wg_a = T;
                ca = C;
            } else {
                nearest_item_by_cost(sa, rsa, wg_a, ca);
            }
            if (se >= C) {
                wg_e = T;
                ce = C;
            } else {
                nearest_item_by_cost(se, rse, wg_e, ce);
            }
        }
        g0 = g1 = wg_a;
        if (ce > ca) {
            const int cw0 = ca + (ce - ca) * wave / NW, cw1 = ca + (ce - ca) * (wave + 1) / NW;
            int rc0, rc1;
            row_of2_in(s_cpre, min(cw0, C - 1), min(cw1, C - 1), rc0, rc1);
            g0 = cw0 >= ce ? wg_e : tile_at_cost(cw0, rc0);
            g1 = cw1 >= ce ? wg_e : tile_at_cost(cw1, rc1);
        }
    }
    // rows of this wavefront's first and last tiles
    if (g1 > g0) row_of2(g0, g1 - 1, rg0, rg1);
    }
    // each wavefront's first tile (and the workgroup's end): a wavefront whose
    // range starts inside an item finds there the one holding the tile before
    s_wstart[wave] = g0;
    if (wave == NW - 1) s_wstart[NW] = g1;
    s_ready[wave] = 0;
    const int ntiles = g1 - g0;

    // ---- fused append: the wavefront holding the last tile of (b, h) -- the
    // only one that reads the block of position L_b - 1 for head h -- writes
    // b's new token for head h there before it loads that tile (unplanned
    // launches: before loading anything; planned ones: below).  A wavefront's
    // vector memory accesses to one address are performed in order, so its
    // later K/V loads of that block return the new token without a wait.
    // A multi-query row's q tokens, at positions L - q .. L - 1, may span
    // tiles and are read by the wavefronts of both chunks of query columns:
    // every wavefront that loads a tile of KV head h holding one of those
    // positions writes all q tokens of head h first (the same bytes
    // whichever wavefront writes them, so the others' stores change nothing
    // it reads).
    constexpr int IB = KIND == kF32 ? 4 : 2;              // input element bytes
    // multi-query row r: whether tiles g0 .. g1 - 1 hold a tile of KV head h
    // with one of its query positions.  Partitions p start at multiples of
    // PS and their tiles jj at multiples of TT within them; the tile number
    // follows the multi-query order (KV head, partition, chunk).
    auto multi_holds = [&](int r, int h) {
        const int th = row_head_tiles(r), base = s_tpre[r];
        const int L = s_len[r], x0 = L - (s_aux[r] & 0xFF);
        const int nch = row_heads(r) / Hkv, n = row_items(r);
        const int rem = th - (n - 1) * tpi, hb = nch * th, full = (n - 1) * nch * tpi;
        for (int p = x0 / PS; p <= (L - 1) / PS; ++p) {
            const int pb = p * PS;
            const int j_lo = (max(x0, pb) - pb) / TT, j_hi = (min(L, pb + PS) - 1 - pb) / TT;
            for (int ch = 0; ch < nch; ++ch) {
                const int t0 = base + h * hb + (p < n - 1 ? p * nch * tpi + ch * tpi : full + ch * rem);
                if (t0 + j_lo < g1 && t0 + j_hi >= g0) return true;
            }
        }
        return false;
    };
    // f(t, h, slot) for each token this wavefront writes, in order; t is the
    // token's row of k_new / v_new (the sequence for one new token per
    // sequence, the query token for multi-query rows)
    auto for_each_append = [&](auto&& f) {
        for (int r = rg0; r <= min(rg1, B - 1); ++r) {
            const int th = row_head_tiles(r);
            if (th == 0) continue;
            if (multi) {
                const int nq = s_aux[r] & 0xFF, q0 = s_aux[r] >> 8, x0 = s_len[r] - nq;
                for (int h = 0; h < Hkv && nq > 0; ++h) {
                    if (!multi_holds(r, h)) continue;
                    for (int i = 0; i < nq; ++i) {
                        const int pos = x0 + i;
                        const int slot = load_invariant(a.new_slots + q0 + i);
                        const int want = load_invariant(a.block_tables + (long)r * a.max_blocks_per_seq +
                                                        pos / kBlock) * kBlock + pos % kBlock;
                        if (slot >= 0 && slot == want) f(q0 + i, h, slot);
                    }
                }
                continue;
            }
            const int base = s_tpre[r];
            // first head whose last tile, base + (h + 1) * th - 1, is at or after g0
            const int x = g0 - base + 1;
            const int h0 = x <= 0 ? 0 : min(Hkv, (x + th - 1) / th - 1);
            if (h0 >= Hkv || base + (h0 + 1) * th - 1 >= g1) continue;
            // only the slot the table gives position L - 1 (the block read below)
            const int lp = max(s_len[r] - 1, 0);
            const int slot = load_invariant(a.new_slots + r);
            const int want = load_invariant(a.block_tables + (long)r * a.max_blocks_per_seq +
                                            lp / kBlock) * kBlock + lp % kBlock;
            if (slot < 0 || slot != want) continue;
            for (int h = h0; h < Hkv; ++h) {
                if (base + (h + 1) * th - 1 >= g1) break;
                f(r, h, slot);
            }
        }
    };
    auto scales = [&](int h, float& ksc, float& vsc) {
        ksc = KIND == kFP8 ? load_invariant(a.k_scale + h) : 1.0f;
        vsc = KIND == kFP8 ? load_invariant(a.v_scale + h) : 1.0f;
    };
    // (a plan's list of tokens is written where the first tile is loaded)
    const bool listed_appends = MODE == kUsePlan && a.new_slots != nullptr && plan_apps >= 0;
    if (MODE != kMakePlan && a.new_slots != nullptr && ntiles > 0) {
        if (!listed_appends && multi) {
            // a row's tokens 512 / D at a time, D / 8 lanes each: one memory
            // round trip per group rather than two per token
            constexpr int CPT = D / 8, TPP = kWave / CPT;
            for (int r = rg0; r <= min(rg1, B - 1); ++r) {
                const int nq = s_aux[r] & 0xFF, q0 = s_aux[r] >> 8, x0 = s_len[r] - nq;
                if (nq <= 0 || row_head_tiles(r) == 0) continue;
                const int32_t* brow = a.block_tables + (long)r * a.max_blocks_per_seq;
                for (int h = 0; h < Hkv; ++h) {
                    if (!multi_holds(r, h)) continue;
                    float ksc, vsc;
                    scales(h, ksc, vsc);
                    for (int i0 = 0; i0 < nq; i0 += TPP) {
                        const int i = i0 + lane / CPT;
                        if (i >= nq) continue;
                        const int pos = x0 + i;
                        const int slot = a.new_slots[q0 + i];
                        const int want = brow[pos / kBlock] * kBlock + pos % kBlock;
                        const long row = ((long)(q0 + i) * Hkv + h) * D * IB;
                        const TokenChunk<KIND> tok = load_token_chunk<KIND, D>(
                            static_cast<const char*>(a.k_new) + row,
                            static_cast<const char*>(a.v_new) + row, lane % CPT);
                        if (slot >= 0 && slot == want)
                            store_token_chunk<KIND, D>(tok, a.k_cache_w, a.v_cache_w, slot / kBlock,
                                                       slot % kBlock, h, Hkv, lane % CPT, ksc, vsc);
                    }
                }
            }
        } else if (!listed_appends) {
            for_each_append([&](int t, int h, int slot) {
                const long row = ((long)t * Hkv + h) * D * IB;
                float ksc, vsc;
                scales(h, ksc, vsc);
                if (lane < D / 8)
                    write_token_chunk<KIND, D>(static_cast<const char*>(a.k_new) + row,
                                               static_cast<const char*>(a.v_new) + row,
                                               a.k_cache_w, a.v_cache_w, slot / kBlock,
                                               slot % kBlock, h, Hkv, lane, ksc, vsc);
            });
        }
    }

    const int g = lane & 15, grp = lane >> 4;
    const long head_stride = (long)kBlock * D * ELEM;              // one (block, head) tile
    const long blk_stride = head_stride * Hkv;

    // Tile cursor: row r, virtual head vh (KV head h, member chunk ch), item
    // p (partition part = p + skip), tile jj of the item; the item covers
    // positions [tb, te) in nti tiles; t0 is its first tile's global number.
    struct Cursor {
        int r, vh, h, ch, nh, p, part, jj, n, tb, te, nti, qmin;
        long t0;
    };
    auto set_item = [&](Cursor& c, int r, int vh, int p, long t0) {
        c.r = r;
        c.vh = vh;
        c.nh = row_heads(r);
        const int chunks = c.nh / Hkv;
        c.h = vh / chunks;
        c.ch = vh - c.h * chunks;
        c.p = p;
        c.part = p + row_skip(r);
        c.n = row_items(r);
        c.tb = c.part * PS;
        c.te = min(s_len[r], c.tb + PS);
        c.nti = (c.te - c.tb + TT - 1) / TT;
        c.qmin = (multi && r < B) ? s_len[r] - (s_aux[r] & 0xFF) : 0x3FFFFFFF;   // first query position
        if (PLAIN) {
            c.h = vh;
            c.ch = 0;
        }
        c.t0 = t0;
    };
    // only called while another tile of this wavefront's run exists
    auto advance = [&](Cursor& c) {
        if (++c.jj < c.nti) return;
        const long t0 = c.t0 + c.nti;
        int r = c.r, vh = c.vh, p = c.p;
        if constexpr (PLAIN || !CI) {               // item, then virtual head, then row
            if (++p == c.n) {
                p = 0;
                if (++vh == c.nh) {
                    vh = 0;
                    do { ++r; } while (s_tpre[r + 1] == s_tpre[r]);    // skip rows without tiles
                }
            }
        } else {
            // skip rows without tiles (bounded: a bad cursor cannot run away)
            auto next_row = [&]() { do { ++r; } while (r < R - 1 && s_tpre[r + 1] == s_tpre[r]); };
            // member chunk, then item, then KV head, then row (the order above)
            const int nch = c.nh / Hkv;
            int h = c.h, ch = c.ch;
            if (++ch == nch) {
                ch = 0;
                if (++p == c.n) {
                    p = 0;
                    if (++h == Hkv) {
                        h = 0;
                        next_row();
                    }
                }
            }
            vh = h * nch + ch;
        }
        c.jj = 0;
        set_item(c, r, vh, p, t0);
    };
    // sequence whose block table a row reads: the row's own, or its group's
    // first member's
    auto table_seq = [&](int r) {
        if (PLAIN || r < B) return r;
        const int sq = load_invariant(a.group_seqs + __builtin_amdgcn_readfirstlane(s_aux[r] >> 16));
        return (sq >= 0 && sq < B) ? sq : 0;
    };

    // cursor at tile g of row r
    auto cursor_at = [&](Cursor& c, int g, int r) __attribute__((always_inline)) {
        int t0, nti, vh, p, jj;
        locate(g, r, t0, nti, vh, p, jj);
        set_item(c, r, vh, p, t0);
        c.jj = jj;
    };

    // ---- the range in processing order: Y, M, X ----------------------------
    // Y = [yb, g1), the first tiles of the item cut at g1; M = the whole items
    // between; X = [g0, xa), the last tiles of the item cut at g0.  Y is
    // computed from the item's start and parked; X continues the state the
    // wavefront before parked.  A range inside one item cut at both ends is
    // one segment that takes the state, continues it and parks it.  Segment k
    // covers tiles [sbk, sek) and starts in row srk.
    int sb0 = 0, se0 = 0, sr0 = 0, sb1 = 0, se1 = 0, sr1 = 0, sb2 = 0, se2 = 0, sr2 = 0;
    bool x_cut = false;       // g0 lies inside an item: X waits for the state of its head
    Cursor cc;                // tile being computed
    if (ntiles > 0) {
        Cursor cx, cy;
        cursor_at(cx, g0, rg0);
        cursor_at(cy, g1 - 1, rg1);
        x_cut = cx.jj != 0;
        const bool y_cut = cy.jj + 1 != cy.nti;
        const int xa = (int)(cx.t0 + cx.nti), yb = (int)cy.t0;
        if (x_cut && y_cut && cx.t0 == cy.t0) {
            sb0 = g0;
            se0 = g1;
            sr0 = rg0;
        } else {
            // the segments that are not empty, in the order Y, M, X (chosen
            // by value: stores through a selected pointer would keep them in
            // scratch memory)
            const int mb = x_cut ? xa : g0, me = y_cut ? yb : g1;
            const bool has_m = mb < me;
            int rm = rg0;
            if (has_m)
                while (s_tpre[rm + 1] <= mb) ++rm;        // the row holding tile mb
            sb0 = y_cut ? yb : has_m ? mb : g0;
            se0 = y_cut ? g1 : has_m ? me : xa;
            sr0 = y_cut ? rg1 : has_m ? rm : rg0;
            sb1 = y_cut && has_m ? mb : g0;
            se1 = y_cut && has_m ? me : xa;
            sr1 = y_cut && has_m ? rm : rg0;
            sb2 = g0;
            se2 = xa;
            sr2 = rg0;
        }
        cursor_at(cc, sb0, sr0);
    }
    // move a cursor to the next tile in processing order; s: its segment.
    // Only called while another tile of this wavefront's range exists.
    // (by value: a conditional over the captured lvalues would select their
    // addresses and keep the whole closure in scratch memory)
    auto pick = [](int k, int v0, int v1, int v2) { return k == 0 ? v0 : k == 1 ? v1 : v2; };
    auto next_tile = [&](Cursor& c, int& s) __attribute__((always_inline)) {
        if (c.t0 + c.jj + 1 == pick(s, se0, se1, se2)) {
            ++s;
            cursor_at(c, pick(s, sb0, sb1, sb2), pick(s, sr0, sr1, sr2));
        } else {
            advance(c);
        }
    };

    // ---- plan launch: record what this prologue found, then stop ----------
    if constexpr (MODE == kMakePlan) {
        int32_t* pl = a.plan_out;
        int32_t* wv = pl + plan_waves_offset(R) + ((long)blockIdx.x * NW + wave) * kPlanWave;
        int w = 0;
        // block ids of the first two tiles, as the load cursor would fetch them
        auto tile_ids = [&](const Cursor& c, int at) {
            const int32_t* btr = a.block_tables + (long)table_seq(c.r) * a.max_blocks_per_seq;
            const int lb = (c.tb + c.jj * TT) / kBlock, last = (c.te - 1) / kBlock;
            if (lane >= at && lane < at + TB) w = btr[min(lb + lane - at, last)];
        };
        if (ntiles > 0) tile_ids(cc, 6);
        if (ntiles > 1) {
            Cursor c1 = cc;
            int s1 = 0;
            next_tile(c1, s1);
            tile_ids(c1, 10);
        }
        const int vals[6] = {g0, g1, wg_a, wg_e, rg0, rg1};
#pragma unroll
        for (int k = 0; k < 6; ++k)
            if (lane == k) w = vals[k];
        // the tokens this wavefront appends, checked against the tables now
        int napp = 0;
        if (a.new_slots != nullptr && ntiles > 0)
            for_each_append([&](int t, int h, int slot) {
                if (napp < kPlanMaxAppends) {
                    if (lane == 16 + 2 * napp) w = t * Hkv + h;
                    if (lane == 17 + 2 * napp) w = slot;
                }
                ++napp;
            });
        if (lane == 14) w = a.new_slots == nullptr || napp > kPlanMaxAppends ? -1 : napp;
        if (lane < kPlanWave) wv[lane] = w;
        if (blockIdx.x == 0) {
            for (int r = tid; r < R; r += NT) {
                pl[kPlanHeader + r] = s_len[r];
                pl[kPlanHeader + R + r] = s_aux[r];
                pl[kPlanHeader + 2 * R + r] = s_tpre[r];
            }
            if (tid < kPlanHeader) {
                const int hdr[kPlanHeader] = {kPlanMagic, B, Hkv, PS, a.max_partitions, TT,
                                              (int)gridDim.x, NW, a.max_blocks_per_seq, a.split,
                                              T, D, R, row_kind, a.new_slots != nullptr, 0};
                int v = 0;
#pragma unroll
                for (int k = 0; k < kPlanHeader; ++k)
                    if (tid == k) v = hdr[k];
                pl[tid] = v;
            }
            if (tid == 0) pl[kPlanHeader + 3 * R] = T;
        }
        return;
    }
    // every wavefront's s_wstart and cleared s_ready are visible from here on
    __syncthreads();

    WaveSoftmax<KIND, D, NC> st;
    typename Ops::Q qop[NC];
    float c = a.scale_log2;
    // this lane's column in query tile n: row of q / the partials (-1: none),
    // query head, and the last position it may see (multi-query rows; others
    // see everything)
    int col_seq[NC], col_hq[NC], col_last[NC];
    // Q operands, column map and score multiplier of item `it`
    auto q_for = [&](const Cursor& it, typename Ops::Q (&qd)[NC], int (&cs)[NC], int (&chq)[NC],
                     int (&cl)[NC], float& cf) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            cs[n] = -1;
            chq[n] = 0;
            cl[n] = 0x3FFFFFFF;
        }
        if (it.r < B && multi) {
            const int aux = __builtin_amdgcn_readfirstlane(s_aux[it.r]);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const int i = it.ch * mpv + n * mpc + g / a.group;
                if (g < mpc * a.group && i < (aux & 0xFF)) {
                    cs[n] = (aux >> 8) + i;
                    chq[n] = it.h * a.group + g % a.group;
                    cl[n] = it.qmin + i;
                }
            }
        } else if (PLAIN || it.r < B) {
            if (g < a.group) {
                cs[0] = it.r;
                chq[0] = it.h * a.group + g;
            }
        } else {
            // this chunk's members, read with scalar loads (no wait on the
            // K/V loads in flight) and handed to their lanes by select
            const int aux = __builtin_amdgcn_readfirstlane(s_aux[it.r]);
            const int first = (aux >> 16) + it.ch * mpv;
            const int cnt = min(mpv, (aux & 0xFFFF) - it.ch * mpv);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const int m = n * mpc + g / a.group;
                int sq = -1;
                for (int k = n * mpc; k < min(cnt, (n + 1) * mpc); ++k) {
                    const int v = load_invariant(a.group_seqs + first + k);
                    sq = (m == k) ? v : sq;
                }
                if (g < mpc * a.group && sq >= 0 && sq < B) {
                    cs[n] = sq;
                    chq[n] = it.h * a.group + g % a.group;
                }
            }
        }
        // Every lane loads, so the loads are no branch of their own: a
        // column without a query reads row 0 (it is never written, and no
        // column's arithmetic reads another's).
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const QT* qrow = reinterpret_cast<const QT*>(a.q) +
                             ((long)max(cs[n], 0) * a.num_heads + chq[n]) * D;
            Ops::load_q(qd[n], qrow, true, lane);
        }
        cf = a.scale_log2;
        if (KIND == kFP8) cf *= load_invariant(a.k_scale + it.h);
    };
    // The load cursor enters each item (row, virtual head) one or two tiles
    // before the compute cursor does; the item's Q operand is loaded then,
    // into one prefetch slot, so its latency stays off the compute path.  The
    // slot holds one item: when the load cursor enters a second item before
    // the compute cursor has taken the first (one-tile items), that second
    // item's Q is loaded when the compute cursor reaches it.  Items are
    // numbered in the order both cursors enter them.
    // The prefetch is issued before the K/V loads of the tile ahead of the
    // item: those loads are complete before that tile is multiplied, so the
    // prefetched operand is complete when the compute cursor takes it.
    // (one query tile only: two would not fit beside two tiles of K/V)
    constexpr bool kPrefetchQ = NC == 1;
    typename Ops::Q qnext[NC];
    int next_seq[NC], next_hq[NC], next_last[NC], next_ord = -1;
    float next_c = 0.f;
    int load_ord = 0, comp_ord = 0;

    // Split-K partial rows written to HBM while the K/V stream runs cost
    // far more than their bytes (the long-context batch's 17.6 MB of
    // partials took about 40 us; the same stores into 2 KB that stays in
    // L2 took nothing).  So launches whose wavefronts stream long ranges
    // (STAGE) collect each wavefront's rows in LDS and write them when the
    // area is full and once the range is done, two 512-byte rows per store
    // instruction.  A short range (a few items) stores at once: held to its
    // end, its rows would only lengthen the launch's tail.
    constexpr bool kStage = STAGE;
    constexpr int kStageMinTiles = 64;
    const bool stage_on = kStage && ntiles >= kStageMinTiles;
    f32x4* stage_o = nullptr;      // this wavefront's rows (kStageRows x D / 4)
    long* stage_pi = nullptr;      // their partial indices
    float* stage_ml = nullptr;     // their (m, l)
    if constexpr (kStage) {
        __shared__ f32x4 s_stage_o[NW][kStageRows * D / 4];
        __shared__ long s_stage_pi[NW][kStageRows];
        __shared__ float s_stage_ml[NW][kStageRows * 2];
        stage_o = s_stage_o[wave];
        stage_pi = s_stage_pi[wave];
        stage_ml = s_stage_ml[wave];
    }
    int staged = 0;                // rows collected (the same in every lane)
    auto flush_stage = [&]() {
        if constexpr (kStage) {
            for (int k = 0; k < staged; k += 2) {
                const int row = k + (lane >> 5);
                if (row < staged) {
                    const f32x4 v = stage_o[row * (D / 4) + (lane & 31)];
                    *reinterpret_cast<f32x4*>(a.part_out + stage_pi[row] * D + 4 * (lane & 31)) = v;
                }
            }
            for (int row = lane; row < staged; row += kWave) {
                a.part_max[stage_pi[row]] = stage_ml[2 * row];
                a.part_sum[stage_pi[row]] = stage_ml[2 * row + 1];
            }
            staged = 0;
        }
    };

    // write an item's result from st: a split-K partial, or the output rows
    auto finish_item = [&](const Cursor& it) {
        const float vs = (KIND == kFP8) ? load_invariant(a.v_scale + it.h) : 1.0f;
        if constexpr (kStage) {
            if (a.split && stage_on) {
                // plain rows: columns g < G hold the item's query heads
                const int cols = a.group;
                if (staged + cols > kStageRows) flush_stage();
                const float lt = sum_over_groups(st.l[0]);
                if (g < cols) {
                    const int row = staged + g;
                    const float inv = vs / lt;
#pragma unroll
                    for (int t = 0; t < NVT; ++t) stage_o[row * (D / 4) + 4 * t + grp] = st.o[0][t] * inv;
                    if (grp == 0) {
                        stage_pi[row] = ((long)col_seq[0] * a.num_heads + col_hq[0]) * a.max_partitions +
                                        it.part;
                        stage_ml[2 * row] = st.m[0] * kLn2;
                        stage_ml[2 * row + 1] = lt * fast_exp2(st.mr[0] - st.m[0]);   // against the true max
                    }
                }
                staged += cols;
                return;
            }
        }
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const float lt = sum_over_groups(st.l[n]);      // against the reference mr
            // a multi-query column that sees none of the item writes nothing
            if (col_seq[n] < 0 || col_last[n] < it.tb) continue;
            const float inv = vs / lt;
            if (a.split) {
                const long pi =
                    ((long)col_seq[n] * a.num_heads + col_hq[n]) * a.max_partitions + it.part;
                float* po = a.part_out + pi * D;
#pragma unroll
                for (int t = 0; t < NVT; ++t)
                    *reinterpret_cast<f32x4*>(po + 16 * t + 4 * grp) = st.o[n][t] * inv;
                if (grp == 0) {
                    a.part_max[pi] = st.m[n] * kLn2;
                    a.part_sum[pi] = lt * fast_exp2(st.mr[n] - st.m[n]);   // against the true max
                }
            } else {
                const long oi = ((long)col_seq[n] * a.num_heads + col_hq[n]) * D;
#pragma unroll
                for (int t = 0; t < NVT; ++t) {
                    const f32x4 v = st.o[n][t] * inv;
                    const int d = 16 * t + 4 * grp;
                    if (KIND == kF32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oi + d) = v;
                    } else {
                        u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + oi + d) = pk;
                    }
                }
            }
        }
    };
    // Hand the running state of the item cut at this wavefront's end to the
    // one that continues it.  A wavefront's LDS writes are performed in
    // order, so once the flag is seen the state is there; the compiler-only
    // fences keep the stores (and, on the taking side, the loads) on their
    // side of the flag without waiting for the K/V loads in flight.  The
    // flag is a relaxed workgroup-scope atomic so that it stays an LDS access:
    // a volatile access through a generic pointer becomes a flat one, which
    // the compiler follows with a wait on every vector memory load in flight.
    auto park = [&]() __attribute__((always_inline)) {
        SegSlot<NVT, NC>& sl = s_seg[wave];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) sl.o[n][t][lane] = st.o[n][t];
            sl.m[n][lane] = st.m[n];
            sl.mr[n][lane] = st.mr[n];
            sl.l[n][lane] = st.l[n];
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(&s_ready[wave], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Take the state of the item cut at g0 from the wavefront holding tile
    // g0 - 1 (the last one before this with a non-empty range; wave 0's range
    // starts at an item).  That wavefront parks it after the first segment it
    // computes, which waits on nobody unless it too lies inside this item,
    // and then on a wavefront before it: the chain ends at the item's head.
    // The wait is bounded (about two seconds, far beyond any item's time):
    // should a damaged plan ever send a range into an item nobody parks, the
    // item comes out NaN instead of the wavefront spinning forever.
    auto take = [&]() __attribute__((always_inline)) {
        int from = max(wave - 1, 0);
        while (from > 0 && s_wstart[from] >= g0) --from;
        bool ok = from < wave;
        for (int spin = 0;
             ok && __hip_atomic_load(&s_ready[from], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
             ++spin) {
            if (spin == (1 << 26)) ok = false;
            __builtin_amdgcn_s_sleep(1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const SegSlot<NVT, NC>& sl = s_seg[from];
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int n = 0; n < NC; ++n) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
                const f32x4 v = sl.o[n][t][lane];
                st.o[n][t] = ok ? v : f32x4{nan, nan, nan, nan};
            }
            st.m[n] = ok ? sl.m[n][lane] : nan;
            st.mr[n] = ok ? sl.mr[n][lane] : nan;
            st.l[n] = ok ? sl.l[n][lane] : nan;
        }
    };

    if (ntiles > 0) {
        Cursor lc = cc;     // tile being loaded (one ahead)
        int ls = 0, cs = 0; // segments of the load and compute cursors
        int nloaded = 0;
        int phys[TB];
        const int32_t* bt = a.block_tables + (long)table_seq(lc.r) * a.max_blocks_per_seq;
        auto fetch_ids = [&]() {
            const int lb = __builtin_amdgcn_readfirstlane((lc.tb + lc.jj * TT) / kBlock);
            const int last = __builtin_amdgcn_readfirstlane((lc.te - 1) / kBlock);
#pragma unroll
            for (int j = 0; j < TB; ++j) phys[j] = load_invariant(bt + min(lb + j, last));
        };
        // The plan's list of the tokens this wavefront appends (D / 8 lanes
        // carry one token, so a register set holds 512 / D): their rows are
        // loaded before anything else.  The stores must precede the loads of
        // the tile holding the token (the last tile of a listed (row, KV
        // head), or the first tile holding a query position of a
        // multi-query row), which then reads it back.  The plain kernel issues them just
        // before that tile's loads -- usually tiles later, when the rows have
        // long arrived, so the stream never waits for them.  The wide kernels
        // have no registers to hold the rows that long: they store as soon as
        // the rows arrive, after the first tile's loads (before them when the
        // first tile holds a token).
        constexpr bool kDeferStores = NC == 1;
        constexpr int CPT = D / 8, TPP = kWave / CPT;
        constexpr int NP = (kPlanMaxAppends + TPP - 1) / TPP;
        TokenChunk<KIND> tok[NP];
        int t_rh[NP], t_slot[NP];
        const bool listed = listed_appends && plan_apps > 0;
        bool stored = !listed;
        if (listed) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int ti = j * TPP + lane / CPT;
                int rh = plan_app_rh[0], slot = -1;
#pragma unroll
                for (int i = 0; i < kPlanMaxAppends; ++i)
                    if (i == ti && i < plan_apps) {
                        rh = plan_app_rh[i];
                        slot = plan_app_slot[i];
                    }
                t_rh[j] = rh;
                t_slot[j] = slot;
                const long row = (long)rh * D * IB;
                tok[j] = load_token_chunk<KIND, D>(static_cast<const char*>(a.k_new) + row,
                                                   static_cast<const char*>(a.v_new) + row,
                                                   lane % CPT);
            }
        }
        auto store_all = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                if (j * TPP >= plan_apps) break;
                const int h = t_rh[j] % Hkv, slot = t_slot[j];
                if (slot >= 0) {
                    float ksc, vsc;
                    scales(h, ksc, vsc);
                    store_token_chunk<KIND, D>(tok[j], a.k_cache_w, a.v_cache_w, slot / kBlock,
                                               slot % kBlock, h, Hkv, lane % CPT, ksc, vsc);
                }
            }
            stored = true;
        };
        // the tile under cursor c holds a listed token not stored yet (a
        // multi-query row's tokens may span tiles: any tile holding one of
        // its query positions is taken to hold them all; a token is listed
        // only for a wavefront that loads such a tile, so the first of them
        // comes no later than the token's own)
        auto holds_token = [&](const Cursor& c) __attribute__((always_inline)) {
            if (multi) return !stored && c.tb + (c.jj + 1) * TT > c.qmin;
            if (stored || c.p + 1 != c.n || c.jj + 1 != c.nti) return false;
            bool hit = false;
#pragma unroll
            for (int i = 0; i < kPlanMaxAppends; ++i)
                hit |= i < plan_apps && plan_app_rh[i] == c.r * Hkv + c.h;
            return hit;
        };
        // load the tile under the load cursor and move the cursor on; the
        // next tile's block ids and (entering an item) Q go out first
        // FIRST: the launch's first load, whose successor's block ids a plan holds
        auto issue = [&](typename Ops::Regs& r, auto first) {
            const bool store_now = kDeferStores && holds_token(lc);
            const long hoff = (long)lc.h * head_stride;
            int ph[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) ph[j] = phys[j];
            if (++nloaded < ntiles) {
                const int orow = lc.r, ovh = lc.vh;
                next_tile(lc, ls);
                if (lc.r != orow)
                    bt = a.block_tables + (long)table_seq(lc.r) * a.max_blocks_per_seq;
                if constexpr (MODE == kUsePlan && decltype(first)::value) {
#pragma unroll
                    for (int j = 0; j < TB; ++j) phys[j] = plan_ids[1][j];
                } else {
                    fetch_ids();
                }
                if (kPrefetchQ && (lc.r != orow || lc.vh != ovh)) {
                    ++load_ord;
                    if (next_ord <= comp_ord) {
                        q_for(lc, qnext, next_seq, next_hq, next_last, next_c);
                        next_ord = load_ord;
                    }
                }
            }
            if (store_now) store_all();
            Ops::load(r, a.k_cache + hoff, a.v_cache + hoff, blk_stride, ph, lane);
        };
        int ncomputed = 0;
        // entering a tile: X's first tile takes the parked state, an item's
        // first tile starts from scratch, any other continues
        auto enter = [&]() __attribute__((always_inline)) {
            if (x_cut && cc.t0 + cc.jj == g0) take();
            else if (cc.jj == 0) st.init();
        };
        auto compute = [&](typename Ops::Regs& r) {
            const int t0 = cc.tb + cc.jj * TT;
            const int nvalid = cc.te - t0;
            int limit[NC];
#pragma unroll
            for (int n = 0; n < NC; ++n) limit[n] = min(col_last[n] - t0, TT);
            st.step(r, qop, c, nvalid, limit, nvalid < TT || t0 + TT - 1 > cc.qmin, lane);
            ++ncomputed;
            const bool item_done = cc.jj + 1 == cc.nti;
            const bool seg_done = cc.t0 + cc.jj + 1 == pick(cs, se0, se1, se2);
            if (item_done) finish_item(cc);
            else if (seg_done) park();                  // continued by a later wavefront
            if (ncomputed == ntiles) return;
            if (item_done || seg_done) {
                const int orow = cc.r, ovh = cc.vh;
                next_tile(cc, cs);
                enter();
                if (cc.r != orow || cc.vh != ovh) {
                    if (kPrefetchQ && ++comp_ord == next_ord) {
#pragma unroll
                        for (int n = 0; n < NC; ++n) {
                            qop[n] = qnext[n];
                            col_seq[n] = next_seq[n];
                            col_hq[n] = next_hq[n];
                            col_last[n] = next_last[n];
                        }
                        c = next_c;
                    } else {
                        q_for(cc, qop, col_seq, col_hq, col_last, c);
                    }
                }
            } else {
                advance(cc);
            }
        };

        q_for(cc, qop, col_seq, col_hq, col_last, c);
        if constexpr (MODE == kUsePlan) {
#pragma unroll
            for (int j = 0; j < TB; ++j) phys[j] = plan_ids[0][j];
        } else {
            fetch_ids();
        }
        typename Ops::Regs ra, rb;
        // tile i is computed while tile i + 1 is in flight
        if (!kDeferStores && holds_token(cc)) store_all();
        issue(ra, std::true_type{});
        if (!kDeferStores && !stored) store_all();
        enter();
        while (true) {
            if (nloaded < ntiles) {
                issue(rb, std::false_type{});
                compute(ra);
            } else {
                compute(ra);
                break;
            }
            if (nloaded < ntiles) {
                issue(ra, std::false_type{});
                compute(rb);
            } else {
                compute(rb);
                break;
            }
        }
        flush_stage();
    }
}

// Launches of plain rows at head size 128 whose bound on tiles per wavefront
// reaches this take the kernel that collects split-K rows in LDS.
constexpr long kStageBoundTiles = 128;

template <int KIND, int D, int NC, bool PLAIN, int MODE = kRun, bool CI = false>
static hipError_t launch_decode(const DecodeArgs& a, long max_tiles, hipStream_t stream) {
    constexpr int NW = 4;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // one workgroup of 4 waves per CU and wave slot; fewer for small problems.
    // Plain rows use 7/8 of that (the same count on each of the 8 XCDs):
    // fewer concurrent streams read the pool faster there (Qwen2.5-3B-shaped
    // batch 30.7 -> 30.3 us in a same-box A/B, long context 377 -> 376 us),
    // while the wide kernels lose by it.
    long grid = (long)cus * waves_per_simd(KIND, D);
    if constexpr (PLAIN) grid = grid * 7 / 8;
    grid = std::min(grid, (max_tiles + NW - 1) / NW);
    grid = std::max(grid, 1L);
    if constexpr (PLAIN && D == 128 && MODE != kMakePlan) {
        if (a.split && max_tiles / (grid * NW) >= kStageBoundTiles) {
            hipLaunchKernelGGL((decode_kernel<KIND, D, NW, NC, PLAIN, MODE, CI, true>),
                               dim3((unsigned)grid), dim3(NW * kWave), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((decode_kernel<KIND, D, NW, NC, PLAIN, MODE, CI>), dim3((unsigned)grid), dim3(NW * kWave), 0,
                       stream, a);
    return hipGetLastError();
}

// items_bound: an upper bound on (row, virtual head, partition) items; wide:
// two 16-column query tiles per wavefront (group and multi-query rows)
static pa_status_t run_decode(const DecodeArgs& a, pa_dtype_t cache_dtype, int head_dim,
                              long items_bound, bool wide, hipStream_t stream) {
    hipError_t e = hipSuccess;
    const int kind = cache_kind(cache_dtype);
    auto tiles = [&](int tt) { return items_bound * ((a.partition_size + tt - 1) / tt); };
    // tile numbers are 32-bit in the kernel
    if (tiles(16) > 0x7fffffffL) return PA_ERR_UNSUPPORTED;
    // multi-query rows take the chunk-inner tile order (CI)
    const bool ci = a.query_start_loc != nullptr;
#define PA_WIDE(K, DD, TT, CIV)                                                               \
    (a.plan_out ? launch_decode<K, DD, 2, false, kMakePlan, CIV>(a, tiles(TT), stream)        \
     : a.plan   ? launch_decode<K, DD, 2, false, kUsePlan, CIV>(a, tiles(TT), stream)         \
                : launch_decode<K, DD, 2, false, kRun, CIV>(a, tiles(TT), stream))
#define PA_LAUNCH(K, DD, TT)                                                          \
    (wide ? (ci ? PA_WIDE(K, DD, TT, true) : PA_WIDE(K, DD, TT, false))              \
          : (a.plan_out ? launch_decode<K, DD, 1, true, kMakePlan>(a, tiles(TT), stream)  \
             : a.plan   ? launch_decode<K, DD, 1, true, kUsePlan>(a, tiles(TT), stream)   \
                        : launch_decode<K, DD, 1, true>(a, tiles(TT), stream)))
    if (kind == kBF16 && head_dim == 128) e = PA_LAUNCH(kBF16, 128, 32);
    else if (kind == kBF16 && head_dim == 64) e = PA_LAUNCH(kBF16, 64, 32);
    else if (kind == kFP8 && head_dim == 128) e = PA_LAUNCH(kFP8, 128, 64);
    else if (kind == kFP8 && head_dim == 64) e = PA_LAUNCH(kFP8, 64, 64);
    else if (kind == kF32 && head_dim == 128) e = PA_LAUNCH(kF32, 128, 16);
    else if (kind == kF32 && head_dim == 64) e = PA_LAUNCH(kF32, 64, 16);
    else return PA_ERR_UNSUPPORTED;
#undef PA_LAUNCH
#undef PA_WIDE
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Split-K partitions (partition_size > 0), or one item covering every
// position a block-table row can address.
static pa_status_t set_partitioning(DecodeArgs& a, int partition_size, int max_partitions,
                                    int max_blocks_per_seq) {
    if (partition_size > 0) {
        if (partition_size % kBlock) return PA_ERR_ARG;
        if (max_partitions < 1) return PA_ERR_ARG;
        a.partition_size = partition_size;
        a.max_partitions = max_partitions;
        a.split = 1;
    } else {
        a.partition_size = max_blocks_per_seq * kBlock;
        a.max_partitions = 1;
        a.split = 0;
    }
    return PA_OK;
}

static long decode_grid_cap(pa_dtype_t cache_dtype, int head_dim) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return (long)cus * waves_per_simd(cache_kind(cache_dtype), head_dim);
}

// Validation and argument packing shared by pa_decode and pa_decode_cascade.
static pa_status_t pack_decode(DecodeArgs& a, void* out, const void* q, pa_dtype_t q_dtype,
                               const void* k_cache, const void* v_cache, pa_dtype_t cache_dtype,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t batch, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float scale, int32_t partition_size, int32_t max_partitions,
                               float* part_max, float* part_sum, float* part_out) {
    pa_status_t st = check_attention_shape(q_dtype, cache_dtype, k_scale, v_scale, num_heads,
                                           num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (batch < 0 || max_blocks_per_seq < 1 || partition_size < 0) return PA_ERR_ARG;
    if (batch == 0) return PA_OK;          // nothing to do; the caller returns
    if (batch > kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_ARG;
    if (!std::isfinite(scale)) return PA_ERR_ARG;
    a = DecodeArgs{};
    a.out = out;
    a.q = q;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.part_out = part_out;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.scale_log2 = scale * kLog2e;
    if (partition_size > 0 && (!part_max || !part_sum || !part_out)) return PA_ERR_ARG;
    if (partition_size == 0 && !out) return PA_ERR_ARG;
    return set_partitioning(a, partition_size, max_partitions, max_blocks_per_seq);
}

// Cascade rows: validation, the group fields and the item bound the grid is
// sized by (batch > 0).
static pa_status_t set_cascade(DecodeArgs& a, const int32_t* group_start, const int32_t* group_seqs,
                               const int32_t* group_prefix_lens, int num_groups,
                               int max_group_size, long& items) {
    if (num_groups < 0 || max_group_size < 0 || max_group_size > 0xFFFF) return PA_ERR_ARG;
    if (num_groups > 0 && (!group_start || !group_seqs || !group_prefix_lens)) return PA_ERR_ARG;
    if ((long)a.batch + num_groups > kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
    a.group_start = group_start;
    a.group_seqs = group_seqs;
    a.group_prefix_lens = group_prefix_lens;
    a.num_groups = num_groups;
    const int mpv = 2 * (16 / a.group);                       // members per virtual head
    const long chunks = (max_group_size + mpv - 1) / mpv;
    items = ((long)a.batch + (long)num_groups * chunks) * a.num_kv_heads * a.max_partitions;
    return PA_OK;
}

// Multi-query rows: validation, the query map and the item bound (batch > 0;
// `none` when no sequence has a query token).
static pa_status_t set_multi(DecodeArgs& a, const int32_t* query_start_loc, int max_query_len,
                             long& items, bool& none) {
    if (max_query_len < 0) return PA_ERR_ARG;
    if (max_query_len > kMaxMultiQuery) return PA_ERR_UNSUPPORTED;
    none = max_query_len == 0;
    if (none) return PA_OK;
    if (!query_start_loc) return PA_ERR_ARG;
    a.query_start_loc = query_start_loc;
    const int mpv = 2 * (16 / a.group);                       // query tokens per virtual head
    const long chunks = (max_query_len + mpv - 1) / mpv;
    items = (long)a.batch * chunks * a.num_kv_heads * a.max_partitions;
    return PA_OK;
}

// The fused append's arrays: all three, or none.
static pa_status_t set_append(DecodeArgs& a, const void* k_new, const void* v_new,
                              const int32_t* new_slots, void* k_cache, void* v_cache) {
    const int given = (k_new != nullptr) + (v_new != nullptr) + (new_slots != nullptr);
    if (given != 0 && given != 3) return PA_ERR_ARG;
    if (given == 3) {
        a.k_new = k_new;
        a.v_new = v_new;
        a.new_slots = new_slots;
        a.k_cache_w = static_cast<char*>(k_cache);
        a.v_cache_w = static_cast<char*>(v_cache);
    }
    return PA_OK;
}

// A plan buffer for `rows` rows large enough for every word a launch reads.
static bool plan_fits(size_t plan_bytes, int rows, pa_dtype_t cache_dtype, int head_dim);

}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_decode(void* out, const void* q, pa_dtype_t q_dtype, const void* k_cache,
                                 const void* v_cache, pa_dtype_t cache_dtype, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, float scale,
                                 int32_t partition_size, int32_t max_partitions, float* part_max,
                                 float* part_sum, float* part_out, hipStream_t stream) {
    DecodeArgs a;
    pa_status_t st = pack_decode(a, out, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                 v_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                                 num_heads, num_kv_heads, head_dim, block_size, scale,
                                 partition_size, max_partitions, part_max, part_sum, part_out);
    if (st != PA_OK || batch == 0) return st;
    return run_decode(a, cache_dtype, head_dim, (long)batch * num_kv_heads * a.max_partitions,
                      false, stream);
}

extern "C" pa_status_t pa_decode_append(void* out, const void* q, pa_dtype_t q_dtype,
                                        const void* k_new, const void* v_new,
                                        const int32_t* new_slots, void* k_cache, void* v_cache,
                                        pa_dtype_t cache_dtype, const float* k_scale,
                                        const float* v_scale, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, float scale,
                                        int32_t partition_size, int32_t max_partitions,
                                        float* part_max, float* part_sum, float* part_out,
                                        const int32_t* plan, size_t plan_bytes,
                                        hipStream_t stream) {
    DecodeArgs a;
    pa_status_t st = pack_decode(a, out, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                 v_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                                 num_heads, num_kv_heads, head_dim, block_size, scale,
                                 partition_size, max_partitions, part_max, part_sum, part_out);
    if (st != PA_OK || batch == 0) return st;
    st = set_append(a, k_new, v_new, new_slots, k_cache, v_cache);
    if (st != PA_OK) return st;
    if (plan) {
        // every word the launch may read lies inside the buffer
        if (!plan_fits(plan_bytes, batch, cache_dtype, head_dim)) return PA_ERR_ARG;
        a.plan = plan;
    }
    return run_decode(a, cache_dtype, head_dim, (long)batch * num_kv_heads * a.max_partitions,
                      false, stream);
}

extern "C" pa_status_t pa_decode_cascade(
    const void* q, pa_dtype_t q_dtype, const void* k_new, const void* v_new,
    const int32_t* new_slots, void* k_cache, void* v_cache,
    pa_dtype_t cache_dtype, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t batch, const int32_t* group_start, const int32_t* group_seqs,
    const int32_t* group_prefix_lens, int32_t num_groups, int32_t max_group_size,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    int32_t partition_size, int32_t max_partitions, float* part_max, float* part_sum,
    float* part_out, const int32_t* plan, size_t plan_bytes, hipStream_t stream) {
    if (partition_size <= 0) return PA_ERR_ARG;
    DecodeArgs a;
    pa_status_t st = pack_decode(a, nullptr, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                 v_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                                 num_heads, num_kv_heads, head_dim, block_size, scale,
                                 partition_size, max_partitions, part_max, part_sum, part_out);
    if (st != PA_OK) return st;
    if (num_groups < 0 || max_group_size < 0 || max_group_size > 0xFFFF) return PA_ERR_ARG;
    if (num_groups > 0 && (!group_start || !group_seqs || !group_prefix_lens)) return PA_ERR_ARG;
    if ((long)batch + num_groups > kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
    if (batch == 0) return PA_OK;
    long items = 0;
    st = set_cascade(a, group_start, group_seqs, group_prefix_lens, num_groups, max_group_size, items);
    if (st != PA_OK) return st;
    st = set_append(a, k_new, v_new, new_slots, k_cache, v_cache);
    if (st != PA_OK) return st;
    if (plan) {
        if (!plan_fits(plan_bytes, batch + num_groups, cache_dtype, head_dim)) return PA_ERR_ARG;
        a.plan = plan;
    }
    return run_decode(a, cache_dtype, head_dim, items, true, stream);
}

extern "C" pa_status_t pa_decode_multi(
    const void* q, pa_dtype_t q_dtype, const void* k_new, const void* v_new,
    const int32_t* new_slots, const int32_t* query_start_loc, int32_t max_query_len,
    void* k_cache, void* v_cache, pa_dtype_t cache_dtype, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, int32_t partition_size,
    int32_t max_partitions, float* part_max, float* part_sum, float* part_out,
    const int32_t* plan, size_t plan_bytes, hipStream_t stream) {
    if (partition_size <= 0) return PA_ERR_ARG;
    DecodeArgs a;
    pa_status_t st = pack_decode(a, nullptr, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                 v_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                                 num_heads, num_kv_heads, head_dim, block_size, scale,
                                 partition_size, max_partitions, part_max, part_sum, part_out);
    if (st != PA_OK) return st;
    if (max_query_len < 0) return PA_ERR_ARG;
    if (max_query_len > kMaxMultiQuery) return PA_ERR_UNSUPPORTED;
    if (batch == 0 || max_query_len == 0) return PA_OK;
    long items = 0;
    bool none = false;
    st = set_multi(a, query_start_loc, max_query_len, items, none);
    if (st != PA_OK || none) return st;
    st = set_append(a, k_new, v_new, new_slots, k_cache, v_cache);
    if (st != PA_OK) return st;
    if (plan) {
        if (!plan_fits(plan_bytes, batch, cache_dtype, head_dim)) return PA_ERR_ARG;
        a.plan = plan;
    }
    return run_decode(a, cache_dtype, head_dim, items, true, stream);
}

extern "C" size_t pa_decode_plan_bytes(int32_t rows, pa_dtype_t cache_dtype, int32_t head_dim) {
    if (rows < 0 || rows > kMaxDecodeRows || !valid_dtype(cache_dtype)) return 0;
    if (head_dim != 64 && head_dim != 128) return 0;
    return (size_t)(plan_waves_offset(rows) + decode_grid_cap(cache_dtype, head_dim) * 4 * kPlanWave) *
           sizeof(int32_t);
}

namespace pa {
static bool plan_fits(size_t plan_bytes, int rows, pa_dtype_t cache_dtype, int head_dim) {
    const size_t need = pa_decode_plan_bytes(rows, cache_dtype, head_dim);
    return need > 0 && plan_bytes >= need;
}
}  // namespace pa

extern "C" pa_status_t pa_decode_plan(int32_t* plan, size_t plan_bytes, pa_plan_entry_t entry,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t batch,
                                      const int32_t* new_slots,
                                      const int32_t* group_start, const int32_t* group_seqs,
                                      const int32_t* group_prefix_lens, int32_t num_groups,
                                      int32_t max_group_size, const int32_t* query_start_loc,
                                      int32_t max_query_len, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      pa_dtype_t cache_dtype, int32_t partition_size,
                                      int32_t max_partitions, hipStream_t stream) {
    if (entry != PA_PLAN_DECODE_APPEND && entry != PA_PLAN_DECODE_CASCADE &&
        entry != PA_PLAN_DECODE_MULTI)
        return PA_ERR_ARG;
    // the query dtype the cache pairs with; a plan launch reads no Q, K, V or scales
    const pa_dtype_t q_dtype = cache_dtype == PA_DT_F32 ? PA_DT_F32 : PA_DT_BF16;
    const float unused_scale = 1.0f;
    pa_status_t st = check_attention_shape(q_dtype, cache_dtype, &unused_scale, &unused_scale,
                                           num_heads, num_kv_heads, head_dim, kBlock);
    if (st != PA_OK) return st;
    if (batch < 0 || max_blocks_per_seq < 1 || partition_size < 0) return PA_ERR_ARG;
    if (entry != PA_PLAN_DECODE_APPEND && partition_size == 0) return PA_ERR_ARG;
    if (entry == PA_PLAN_DECODE_CASCADE && num_groups < 0) return PA_ERR_ARG;
    if (batch == 0) return PA_OK;
    if (batch > kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
    if (!plan || !block_tables || !context_lens) return PA_ERR_ARG;
    DecodeArgs a = DecodeArgs{};
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    st = set_partitioning(a, partition_size, max_partitions, max_blocks_per_seq);
    if (st != PA_OK) return st;
    long items = (long)batch * num_kv_heads * a.max_partitions;
    int rows = batch;
    if (entry == PA_PLAN_DECODE_CASCADE) {
        st = set_cascade(a, group_start, group_seqs, group_prefix_lens, num_groups, max_group_size,
                         items);
        rows = batch + num_groups;
    } else if (entry == PA_PLAN_DECODE_MULTI) {
        bool none = false;
        st = set_multi(a, query_start_loc, max_query_len, items, none);
        if (st == PA_OK && none) return PA_OK;            // no launch will read it
    }
    if (st != PA_OK) return st;
    if (!plan_fits(plan_bytes, rows, cache_dtype, head_dim)) return PA_ERR_ARG;
    a.new_slots = new_slots;
    a.plan_out = plan;
    return run_decode(a, cache_dtype, head_dim, items, entry != PA_PLAN_DECODE_APPEND, stream);
}
