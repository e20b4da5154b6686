// ne_split.cpp -- host plan of the key-range split of the longest causal row blocks.
//
// With causal masking, row block rb of a (batch, KV head) group visits about rb + 1 key tiles, so
// when a launch holds only one or two row blocks per CU slot the longest blocks finish last while
// most CUs idle.  The plan cuts the blocks rb >= rs into np pieces of contiguous key tiles and
// orders all jobs longest-first; (rs, np) is the choice whose simulated greedy dispatch (each job
// to the slot that frees first, as the hardware dispatcher does) ends earliest, counting a fixed
// cost per job (operand loads, epilogue) and per piece (writing or reading the partial result).
// Plans are cached per shape: they depend only on the shape, never on the data or the device.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "ne_launch.hpp"

namespace ne {
namespace {

constexpr int kCus = 256;            // CUs of the chip the plan is made for
constexpr double kMinGain = 0.8;     // split only if the simulated end drops below this fraction

// Per pass: rows per job, workgroups per CU, most pieces per block, and the costs in steps of
// that pass (one 64-key tile of the block's rows): per job (operand loads, epilogue) and per
// piece of a split block -- the hand-off (partial result through memory, agent-scope release /
// acquire, which write back and invalidate the XCD's L2 and so also cost the other workgroups
// there) measured at several steps' time, so splitting pays only where the unsplit order leaves
// most CUs idle (a group or two per launch), not for a 20% imbalance.
struct Kind {
    int BM, wg, maxp;
    double job, piece;
};
constexpr Kind kKinds[3] = {
    {256, 1, 4, 1.0, 4.0},   // forward: 256 rows x 64 keys per step
    {128, 2, 2, 1.0, 4.0},   // dQ: 128 rows x 64 keys
    {64, 1, 4, 2.0, 16.0},   // dK/dV: 64 keys x 64 rows (four products, about half a forward step);
                             // a 4-way split of the 512-token layer's longest key blocks measured
                             // 28.3 against 24.5 us for single blocks
};

struct Entry {
    int kind, T, G, ngrp, D;
    int njobs, rs, np, nrb;
    std::vector<unsigned short> job;
};

double simulate(const std::vector<double>& cost, int ngrp, int slots) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> q;
    for (int i = 0; i < slots; ++i) q.push(0.0);
    double end = 0.0;
    for (double c : cost)
        for (int g = 0; g < ngrp; ++g) {
            const double t = q.top() + c;
            q.pop();
            q.push(t);
            end = std::max(end, t);
        }
    return end;
}

struct Job {
    double cost;
    int rb, piece;
};

// jobs of one group for (rs, np), longest first (ties: later block first, then piece order)
std::vector<Job> jobs_for(const std::vector<int>& tiles, int rs, int np, const Kind& k) {
    std::vector<Job> j;
    const int nrb = (int)tiles.size();
    for (int rb = 0; rb < nrb; ++rb) {
        if (rb >= rs) {
            const int n = tiles[rb];
            for (int p = 0; p < np; ++p)
                j.push_back({(double)(n * (p + 1) / np - n * p / np) + k.job + k.piece, rb, p});
        } else {
            j.push_back({(double)tiles[rb] + k.job, rb, 0});
        }
    }
    std::stable_sort(j.begin(), j.end(), [](const Job& a, const Job& b) {
        if (a.cost != b.cost) return a.cost > b.cost;
        if (a.rb != b.rb) return a.rb > b.rb;
        return a.piece < b.piece;
    });
    return j;
}

// Steps of each block, indexed so that they grow with the index: forward and dQ, row block rb
// (its causal keys); dK/dV, key block nkb - 1 - rb (its rows from the diagonal on).
std::vector<int> block_steps(int kind, int BM, int64_t TG, int T, int G, int nrb) {
    std::vector<int> tiles(nrb);
    for (int rb = 0; rb < nrb; ++rb) {
        if (kind == kSplitDkdv) {
            const int64_t kb = nrb - 1 - rb;
            tiles[rb] = (int)((TG - kb * 64 * G + 63) / 64);
        } else {
            tiles[rb] = (int)(std::min<int64_t>((int64_t)rb * BM + BM - 1, TG - 1) / G / 64 + 1);
        }
    }
    (void)T;
    return tiles;
}

Entry make_plan(int kind, int T, int G, int ngrp, int D) {
    Kind k = kKinds[kind];
    if (kind == kSplitFwd && D <= 64) { k.BM = 128; k.wg = 3; }   // the forward's D <= 64 variant
    Entry e{kind, T, G, ngrp, D, 0, 0, 1, 0, {}};
    const int64_t TG = (int64_t)T * G;
    const int64_t nrb64 = kind == kSplitDkdv ? ((int64_t)T + 63) / 64 : (TG + k.BM - 1) / k.BM;
    e.nrb = (int)std::min<int64_t>(nrb64, INT32_MAX);
    // dK/dV at head_dim <= 64: its planned variant (two workgroups per CU) is always the one to run,
    // with single key blocks unless a split pays
    const bool w4 = kind == kSplitDkdv && D <= 64;
    const int slots = kCus * (w4 ? 2 : k.wg);
    if (nrb64 > 16383 || (w4 && nrb64 > kMaxSplitJobs)) return e;
    auto singles = [&]() {
        e.njobs = e.nrb;
        e.rs = e.nrb;
        e.np = 1;
        e.job.clear();
        for (int rb = e.nrb - 1; rb >= 0; --rb) e.job.push_back((unsigned short)(rb << 2));
        return e;
    };
    // enough blocks per slot: the longest-first order balances by itself
    if ((int64_t)ngrp * nrb64 > (int64_t)4 * slots) return w4 ? singles() : e;
    const std::vector<int> tiles = block_steps(kind, k.BM, TG, T, G, e.nrb);
    std::vector<double> cost;
    auto eval = [&](const std::vector<Job>& j) {
        cost.clear();
        for (const Job& x : j) cost.push_back(x.cost);
        return simulate(cost, ngrp, slots);
    };
    // dK/dV without a plan runs mirrored pairs of key blocks: equal work per workgroup
    double base;
    if (kind == kSplitDkdv) {
        const int npair = (e.nrb + 1) / 2;
        cost.assign(npair, 0.0);
        for (int i = 0; i < npair; ++i)
            cost[i] = tiles[e.nrb - 1 - i] + (i != e.nrb - 1 - i ? tiles[i] + k.job : 0.0) + k.job;
        base = simulate(cost, ngrp, slots);
    } else {
        base = eval(jobs_for(tiles, e.nrb, 1, k));
    }
    // dK/dV: single key blocks longest-first, none split, need no hand-off -- the first choice when
    // the pairs leave CUs idle
    double ref = base;
    bool single = false;
    if (kind == kSplitDkdv) {
        const double m = eval(jobs_for(tiles, e.nrb, 1, k));
        if (w4 || m < 0.97 * base) { ref = m; single = true; }
    }
    double best = ref;
    int brs = e.nrb, bnp = 1;
    // candidate first split blocks: every block for short lists, else 32 evenly spaced ones
    const int step = std::max(1, e.nrb / 32);
    for (int np = 2; np <= k.maxp; ++np)
        for (int rs = e.nrb - 1; rs >= 0; rs -= step) {
            if (tiles[rs] < 2 * np) break;  // tiles grow with rb: smaller rs only shortens pieces
            if ((int64_t)rs + (int64_t)(e.nrb - rs) * np > kMaxSplitJobs) break;
            const double m = eval(jobs_for(tiles, rs, np, k));
            if (m < best) { best = m; brs = rs; bnp = np; }
        }
    if (bnp == 1 || best > kMinGain * ref)  // not worth the hand-off
        return single ? singles() : e;
    const std::vector<Job> j = jobs_for(tiles, brs, bnp, k);
    e.njobs = (int)j.size();
    e.rs = brs;
    e.np = bnp;
    for (const Job& x : j) e.job.push_back((unsigned short)(x.rb << 2 | x.piece));
    return e;
}

std::mutex g_mu;
std::vector<Entry>* g_cache = nullptr;

}  // namespace

void split_plan(int kind, int T, int G, int ngrp, int D, SplitPlan* out) {
    if (kind == kSplitDq) D = 0;   // the forward and dK/dV plans depend on head_dim (<= 64 or not)
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cache) g_cache = new std::vector<Entry>();  // kept for the process (entries are small)
    const Entry* hit = nullptr;
    for (const Entry& e : *g_cache)
        if (e.kind == kind && e.T == T && e.G == G && e.ngrp == ngrp && (e.D <= 64) == (D <= 64)) hit = &e;
    if (!hit) {
        if (g_cache->size() >= 256) g_cache->erase(g_cache->begin());
        g_cache->push_back(make_plan(kind, T, G, ngrp, D));
        hit = &g_cache->back();
    }
    out->njobs = hit->njobs;
    out->rs = hit->rs;
    out->np = hit->np;
    out->nrb = hit->nrb;
    std::copy(hit->job.begin(), hit->job.end(), out->job);
}

}  // namespace ne
