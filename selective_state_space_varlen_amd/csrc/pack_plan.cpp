// varlen_pack_plan: host-side sequence packer.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "结论与讨论":
// sequences are either packed in arrival order, a pack being sealed when the
// next sequence does not fit (the article measures 19.1% padding this way), or
// a window of pending sequences is sorted and packed greedily (as low as 0.46%).
// The greedy rule taken here is first-fit decreasing inside each window of
// `window` sequences: longest first (ties in arrival order), each into the
// lowest-numbered pack of the window with room, packs sealed at the window's
// end.
//
// First fit runs over a tournament tree whose leaves are the window's packs and
// whose nodes hold the largest remaining room below them; unopened packs hold
// the full capacity, so "leftmost leaf with room >= v" is the first open pack
// that fits, or else the next new pack. A window of w sequences costs
// O(w log w) for the sort and O(w log w) for the placements.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "ssmpack.h"

namespace {

struct FirstFit {
    int leaves = 1;
    std::vector<int32_t> room;  // 1-based heap, room[1] is the root

    void reset(int n, int32_t capacity) {
        leaves = 1;
        while (leaves < n) leaves <<= 1;
        room.assign(2 * (size_t)leaves, capacity);
    }
    // Place v into the leftmost pack with room >= v; returns the pack index.
    // With at most n - 1 earlier placements an unopened leaf always remains,
    // so the root holds room >= v whenever v <= capacity.
    int place(int32_t v) {
        int i = 1;
        while (i < leaves) i = (room[2 * i] >= v) ? 2 * i : 2 * i + 1;
        const int pack = i - leaves;
        room[i] -= v;
        for (i >>= 1; i >= 1; i >>= 1) room[i] = std::max(room[2 * i], room[2 * i + 1]);
        return pack;
    }
};

// Arrival order: a new pack opens when the next sequence does not fit.
int32_t plan_sequential(const int32_t* len, int32_t nseq, int32_t capacity, int32_t* order, int32_t* bounds,
                        int32_t* maxlen) {
    int32_t np = 0;
    int64_t load = 0;
    for (int32_t i = 0; i < nseq; ++i) {
        if (np == 0 || load + len[i] > capacity) {
            bounds[np] = i;
            maxlen[np++] = 0;
            load = 0;
        }
        order[i] = i;
        load += len[i];
        maxlen[np - 1] = std::max(maxlen[np - 1], len[i]);
    }
    bounds[np] = nseq;
    return np;
}

// First-fit decreasing inside each window of `window` sequences.
int32_t plan_local_greedy(const int32_t* len, int32_t nseq, int32_t capacity, int32_t window, int32_t* order,
                          int32_t* bounds, int32_t* maxlen) {
    const int32_t wmax = std::max<int32_t>(1, std::min(window, nseq));
    std::vector<int32_t> idx(wmax), owner(wmax), count(wmax + 1);
    FirstFit ff;
    int32_t np = 0, out = 0;
    bounds[0] = 0;
    for (int64_t w0 = 0; w0 < nseq; w0 += window) {
        const int32_t w = (int32_t)std::min<int64_t>(window, nseq - w0);
        for (int32_t k = 0; k < w; ++k) idx[k] = (int32_t)w0 + k;
        std::stable_sort(idx.begin(), idx.begin() + w, [&](int32_t a, int32_t b) { return len[a] > len[b]; });
        ff.reset(w, capacity);
        int32_t used = 0;
        for (int32_t k = 0; k < w; ++k) {
            owner[k] = ff.place(len[idx[k]]);
            used = std::max(used, owner[k] + 1);
        }
        // group by pack, keeping placement order inside each pack
        std::fill(count.begin(), count.begin() + used + 1, 0);
        for (int32_t k = 0; k < w; ++k) ++count[owner[k] + 1];
        for (int32_t p = 0; p < used; ++p) count[p + 1] += count[p];
        for (int32_t p = 0; p < used; ++p) {
            bounds[np + p + 1] = out + count[p + 1];
            maxlen[np + p] = 0;
        }
        for (int32_t k = 0; k < w; ++k) {
            const int32_t p = owner[k];
            order[out + count[p]++] = idx[k];
            maxlen[np + p] = std::max(maxlen[np + p], len[idx[k]]);
        }
        out += w;
        np += used;
    }
    return np;
}

}  // namespace

extern "C" int varlen_pack_plan(const int32_t* lengths, int32_t nseq, int32_t capacity, int32_t strategy,
                                int32_t window, int32_t* order, int32_t* pack_bounds, int32_t* cu_seqlens,
                                int32_t* max_seqlen, int32_t* n_packs, int64_t* padding) {
    if (nseq < 0 || capacity < 1) return SSMP_ERR_SHAPE;
    if (strategy != SSMP_PACK_SEQUENTIAL && strategy != SSMP_PACK_LOCAL_GREEDY) return SSMP_ERR_UNSUPPORTED;
    if (strategy == SSMP_PACK_LOCAL_GREEDY && window < 1) return SSMP_ERR_SHAPE;
    if (!pack_bounds || !cu_seqlens || !n_packs || !padding) return SSMP_ERR_NULL;
    if (nseq > 0 && (!lengths || !order || !max_seqlen)) return SSMP_ERR_NULL;
    int64_t total = 0;
    for (int32_t i = 0; i < nseq; ++i) {
        if (lengths[i] < 0 || lengths[i] > capacity) return SSMP_ERR_SHAPE;
        total += lengths[i];
    }
    if (total >= (int64_t(1) << 31)) return SSMP_ERR_SHAPE;

    int32_t np;
    if (strategy == SSMP_PACK_SEQUENTIAL) {
        pack_bounds[0] = 0;
        np = plan_sequential(lengths, nseq, capacity, order, pack_bounds, max_seqlen);
    } else {
        try {
            np = plan_local_greedy(lengths, nseq, capacity, window, order, pack_bounds, max_seqlen);
        } catch (const std::bad_alloc&) {
            return SSMP_ERR_SHAPE;  // the window's host scratch does not fit in memory
        }
    }
    cu_seqlens[0] = 0;
    for (int32_t k = 0; k < nseq; ++k) cu_seqlens[k + 1] = cu_seqlens[k] + lengths[order[k]];
    *n_packs = np;
    *padding = (int64_t)np * capacity - total;
    return SSMP_OK;
}
