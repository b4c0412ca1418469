// Token graph and Leiden partition on the host (ckv_leiden_partition,
// ckv_partition_quality).
//
// "CommunityKV: Efficient Long-Context Decoding via Graph Partitioning",
// Figure 1 caption: panel (1) links every prompt token to the earlier tokens
// it attends to most (sinks excluded), panel (2) partitions that graph with the
// Leiden algorithm, panel (3) gives every decoded token edges the same way.
// Figure 2 (left): a resolution parameter sets the community size.  Figure 3
// (left): modularity Q of the partition over generation.  Tables 8 and 9 set
// incremental assignment against re-partitioning the grown graph.  Figure 4:
// the partitioning of each layer is dispatched asynchronously while the GPU
// goes on with later layers, so it runs here, on host threads, one graph per
// task.
//
// The algorithm is not printed on the page; it is written from its
// publication (Traag, Waltman, van Eck, "From Louvain to Leiden: guaranteeing
// well-connected communities", Sci. Rep. 9, 5233, 2019): fast local moving of
// nodes, refinement of each community into well-connected sub-communities,
// aggregation of the refined partition with the unrefined one as the
// aggregate's starting partition, until every community of a level is one
// node.  Where that paper draws at random this code takes fixed choices (the
// queue starts in node order; the best candidate wins, staying on ties, the
// lower community id among equal candidates; a new community, the lowest free
// id, only when strictly better; refinement at theta -> 0, i.e. the best
// strictly positive merge), and all gains are compared as exact integers, so
// the partition is a function of the graph alone.

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <functional>
#include <queue>
#include <thread>
#include <vector>

#include "ckv.h"

namespace {

using i64 = int64_t;

// Undirected graph in CSR form: row v lists (neighbour, weight) in increasing
// neighbour order, a self-loop (aggregate levels) as the entry (v, w).
// Weights, degrees and community totals are at most 2m < 2^30 (the entry
// points refuse larger graphs), so they are held in int32; every product is
// taken in int64.
struct Graph {
    int32_t n = 0;
    std::vector<i64> off;
    std::vector<int32_t> nbr;
    std::vector<int32_t> w;
};

// Level-0 graph of tokens n_sinks .. n_tok-1 (node i = token n_sinks + i): every
// listed edge i -> j adds one to A[i][j] and A[j][i].  Returns false on an edge
// that is not to an earlier-or-later non-sink token other than itself.
bool token_graph(const int32_t *rows, int32_t kappa, int32_t n_tok, int32_t n_sinks, Graph &g) {
    const int32_t n = std::max(0, n_tok - n_sinks);
    g.n = n;
    std::vector<i64> cnt(size_t(n) + 1, 0);
    std::vector<int32_t> outdeg(size_t(n), 0);
    bool backward = true;  // every edge to an earlier token (rows from top-kappa selections)
    for (int32_t i = n_sinks; i < n_tok; ++i)
        for (int32_t e = 0; e < kappa; ++e) {
            const int32_t j = rows[size_t(i) * kappa + e];
            if (j < 0) continue;
            if (j < n_sinks || j >= n_tok || j == i) return false;
            backward = backward && j < i;
            cnt[i - n_sinks + 1]++;
            cnt[j - n_sinks + 1]++;
            outdeg[i - n_sinks]++;
        }
    for (int32_t v = 0; v < n; ++v) cnt[v + 1] += cnt[v];
    std::vector<int32_t> raw(static_cast<size_t>(cnt[n]));
    std::vector<i64> pos(cnt.begin(), cnt.end() - 1);
    for (int32_t i = n_sinks; i < n_tok; ++i)
        for (int32_t e = 0; e < kappa; ++e) {
            const int32_t j = rows[size_t(i) * kappa + e];
            if (j < 0) continue;
            const int32_t a = i - n_sinks, b = j - n_sinks;
            raw[pos[a]++] = b;
            raw[pos[b]++] = a;
        }
    g.off.assign(size_t(n) + 1, 0);
    g.nbr.clear();
    g.w.clear();
    g.nbr.reserve(raw.size());
    g.w.reserve(raw.size());
    for (int32_t v = 0; v < n; ++v) {
        // With backward edges only, v's list is its own row's targets (all
        // below v, filled first) followed by the tokens that name v (all
        // above v, filled in increasing order): only the first part needs
        // sorting.
        std::sort(raw.begin() + cnt[v], raw.begin() + (backward ? cnt[v] + outdeg[v] : cnt[v + 1]));
        for (i64 e = cnt[v]; e < cnt[v + 1]; ++e) {
            if (!g.nbr.empty() && i64(g.nbr.size()) > g.off[v] && g.nbr.back() == raw[e]) {
                g.w.back() += 1;
            } else {
                g.nbr.push_back(raw[e]);
                g.w.push_back(1);
            }
        }
        g.off[v + 1] = i64(g.nbr.size());
    }
    return true;
}

std::vector<int32_t> degrees(const Graph &g) {
    std::vector<int32_t> k(g.n, 0);
    for (int32_t v = 0; v < g.n; ++v)
        for (i64 e = g.off[v]; e < g.off[v + 1]; ++e) k[v] += g.w[e];
    return k;
}

using MinHeap = std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>>;

struct Params {
    i64 two_m, gnum, gden;
};

// Fast local moving.  The value of community C for node v (v left out of
// every community) is A(v, C) * 2m * den - num * k_v * K_C; v goes to the
// community of largest value.
void move_nodes(const Graph &g, const std::vector<int32_t> &k, const Params &P, std::vector<int32_t> &comm,
                MinHeap &empty) {
    const int32_t n = g.n;
    std::vector<int32_t> Kc(n, 0), to(n, 0);
    std::vector<int32_t> size(n, 0), touched;
    std::vector<uint8_t> queued(n, 1), mark(n, 0);
    for (int32_t v = 0; v < n; ++v) {
        Kc[comm[v]] += k[v];
        size[comm[v]]++;
    }
    // ring buffer: a node is in the queue at most once
    std::vector<int32_t> ring(size_t(n) + 1);
    size_t head = 0, tail = 0;
    const size_t cap = size_t(n) + 1;
    for (int32_t v = 0; v < n; ++v) ring[tail++] = v;
    while (head != tail) {
        const int32_t v = ring[head];
        head = (head + 1) % cap;
        queued[v] = 0;
        const int32_t D = comm[v];
        touched.clear();
        for (i64 e = g.off[v]; e < g.off[v + 1]; ++e) {
            const int32_t u = g.nbr[e];
            if (u == v) continue;
            const int32_t c = comm[u];
            if (!mark[c]) {
                mark[c] = 1;
                touched.push_back(c);
            }
            to[c] += g.w[e];
        }
        const i64 kv = k[v];
        int32_t best = D;
        i64 best_s = i64(to[D]) * P.two_m * P.gden - P.gnum * kv * (Kc[D] - kv);
        for (int32_t c : touched) {
            if (c == D) continue;
            const i64 s = i64(to[c]) * P.two_m * P.gden - P.gnum * kv * Kc[c];
            if (s > best_s || (s == best_s && best != D && c < best)) {
                best = c;
                best_s = s;
            }
        }
        for (int32_t c : touched) {
            to[c] = 0;
            mark[c] = 0;
        }
        if (best_s < 0 && !empty.empty()) {  // never empty then: D holds another node, so an id is free
            best = empty.top();
            empty.pop();
        }
        if (best == D) continue;
        Kc[D] -= kv;
        if (--size[D] == 0) empty.push(D);
        Kc[best] += kv;
        size[best]++;
        comm[v] = best;
        for (i64 e = g.off[v]; e < g.off[v + 1]; ++e) {
            const int32_t u = g.nbr[e];
            if (u != v && comm[u] != best && !queued[u]) {
                ring[tail] = u;
                tail = (tail + 1) % cap;
                queued[u] = 1;
            }
        }
    }
}

// Refinement: inside every community S each node starts alone; a node
// well-connected to S that is still alone joins the adjacent refined
// community R inside S, itself well-connected to S, of largest strictly
// positive value A(v, R) * 2m * den - num * k_v * K_R.  Refined ids are node
// indices.
std::vector<int32_t> refine(const Graph &g, const std::vector<int32_t> &k, const Params &P,
                            const std::vector<int32_t> &comm) {
    const int32_t n = g.n;
    std::vector<int32_t> ref(n), size(n, 1), touched;
    std::vector<int32_t> Kr(k), ext(n, 0), inside(n, 0), to(n, 0);
    std::vector<uint8_t> mark(n, 0);
    for (int32_t v = 0; v < n; ++v) ref[v] = v;
    // nodes grouped by community, increasing node order inside each
    std::vector<int32_t> start(size_t(n) + 1, 0), order(n);
    for (int32_t v = 0; v < n; ++v) start[comm[v] + 1]++;
    for (int32_t c = 0; c < n; ++c) start[c + 1] += start[c];
    {
        std::vector<int32_t> at(start.begin(), start.end() - 1);
        for (int32_t v = 0; v < n; ++v) order[at[comm[v]]++] = v;
    }
    for (int32_t C = 0; C < n; ++C) {
        const int32_t s0 = start[C], s1 = start[C + 1];
        if (s0 == s1) continue;
        i64 KS = 0;
        for (int32_t i = s0; i < s1; ++i) {
            const int32_t v = order[i];
            KS += k[v];
            int32_t in = 0;
            for (i64 e = g.off[v]; e < g.off[v + 1]; ++e)
                if (g.nbr[e] != v && comm[g.nbr[e]] == C) in += g.w[e];
            inside[v] = in;
            ext[v] = in;
        }
        for (int32_t i = s0; i < s1; ++i) {
            const int32_t v = order[i];
            const i64 kv = k[v];
            if (i64(inside[v]) * P.two_m * P.gden < P.gnum * kv * (KS - kv)) continue;
            if (size[ref[v]] != 1) continue;
            touched.clear();
            for (i64 e = g.off[v]; e < g.off[v + 1]; ++e) {
                const int32_t u = g.nbr[e];
                if (u == v || comm[u] != C) continue;
                const int32_t r = ref[u];
                if (!mark[r]) {
                    mark[r] = 1;
                    touched.push_back(r);
                }
                to[r] += g.w[e];
            }
            int32_t best = -1;
            i64 best_g = 0;
            for (int32_t r : touched) {
                if (r == ref[v]) continue;
                if (i64(ext[r]) * P.two_m * P.gden < P.gnum * Kr[r] * (KS - Kr[r])) continue;
                const i64 gain = i64(to[r]) * P.two_m * P.gden - P.gnum * kv * Kr[r];
                if (gain > best_g || (gain == best_g && best >= 0 && r < best)) {
                    best = r;
                    best_g = gain;
                }
            }
            const int32_t to_best = best >= 0 ? to[best] : 0;
            for (int32_t r : touched) {
                to[r] = 0;
                mark[r] = 0;
            }
            if (best < 0) continue;
            const int32_t old = ref[v];
            ext[best] += inside[v] - 2 * to_best;
            Kr[best] += kv;
            size[best]++;
            Kr[old] = 0;
            size[old] = 0;
            ext[old] = 0;
            ref[v] = best;
        }
    }
    return ref;
}

// Aggregate graph of the refined communities (numbered by refined id in
// increasing order), its starting partition (the rank of each aggregate
// node's community of `comm` among the communities in use) and the map from
// old node to aggregate node.
void aggregate(const Graph &g, const std::vector<int32_t> &ref, const std::vector<int32_t> &comm, Graph &out,
               std::vector<int32_t> &start_comm, std::vector<int32_t> &node_map) {
    const int32_t n = g.n;
    std::vector<int32_t> rank(n, -1), crank(n, -1);
    int32_t na = 0, nc = 0;
    {
        std::vector<uint8_t> used(n, 0), cused(n, 0);
        for (int32_t v = 0; v < n; ++v) {
            used[ref[v]] = 1;
            cused[comm[v]] = 1;
        }
        for (int32_t r = 0; r < n; ++r) {
            if (used[r]) rank[r] = na++;
            if (cused[r]) crank[r] = nc++;
        }
    }
    node_map.assign(n, 0);
    start_comm.assign(na, 0);
    for (int32_t v = 0; v < n; ++v) {
        node_map[v] = rank[ref[v]];
        start_comm[node_map[v]] = crank[comm[v]];
    }
    // members of each aggregate node
    std::vector<int32_t> mstart(size_t(na) + 1, 0), mem(n);
    for (int32_t v = 0; v < n; ++v) mstart[node_map[v] + 1]++;
    for (int32_t a = 0; a < na; ++a) mstart[a + 1] += mstart[a];
    {
        std::vector<int32_t> at(mstart.begin(), mstart.end() - 1);
        for (int32_t v = 0; v < n; ++v) mem[at[node_map[v]]++] = v;
    }
    out.n = na;
    out.off.assign(size_t(na) + 1, 0);
    out.nbr.clear();
    out.w.clear();
    std::vector<int32_t> acc(na, 0);
    std::vector<uint8_t> mark(na, 0);
    std::vector<int32_t> touched;
    for (int32_t a = 0; a < na; ++a) {
        touched.clear();
        for (int32_t i = mstart[a]; i < mstart[a + 1]; ++i) {
            const int32_t v = mem[i];
            for (i64 e = g.off[v]; e < g.off[v + 1]; ++e) {
                const int32_t b = node_map[g.nbr[e]];
                if (!mark[b]) {
                    mark[b] = 1;
                    touched.push_back(b);
                }
                acc[b] += g.w[e];
            }
        }
        std::sort(touched.begin(), touched.end());
        for (int32_t b : touched) {
            out.nbr.push_back(b);
            out.w.push_back(acc[b]);
            acc[b] = 0;
            mark[b] = 0;
        }
        out.off[a + 1] = i64(out.nbr.size());
    }
}

// Leiden on the level-0 graph; labels numbered in order of first node.
// Returns the number of communities.
int32_t leiden(const Graph &g0, i64 gnum, i64 gden, int32_t *labels) {
    const int32_t n0 = g0.n;
    std::vector<int32_t> k = degrees(g0);
    i64 two_m = 0;
    for (int32_t x : k) two_m += x;
    std::vector<int32_t> node_of(n0);
    for (int32_t i = 0; i < n0; ++i) node_of[i] = i;
    std::vector<int32_t> comm(node_of);
    if (two_m > 0) {
        const Params P{two_m, gnum, gden};
        Graph level;
        const Graph *cur = &g0;
        MinHeap empty;
        while (true) {
            move_nodes(*cur, k, P, comm, empty);
            int32_t n_comm = 0;
            {
                std::vector<uint8_t> used(cur->n, 0);
                for (int32_t c : comm) n_comm += !used[c], used[c] = 1;
            }
            if (n_comm == cur->n) break;
            std::vector<int32_t> ref = refine(*cur, k, P, comm);
            int32_t n_ref = 0;
            {
                std::vector<uint8_t> used(cur->n, 0);
                for (int32_t r : ref) n_ref += !used[r], used[r] = 1;
            }
            if (n_ref == cur->n) break;
            Graph next;
            std::vector<int32_t> start, node_map;
            aggregate(*cur, ref, comm, next, start, node_map);
            for (int32_t &a : node_of) a = node_map[a];
            level = std::move(next);
            cur = &level;
            comm = std::move(start);
            k = degrees(level);
            empty = MinHeap();
            for (int32_t c = n_comm; c < level.n; ++c) empty.push(c);
        }
    }
    // communities in order of their first node
    std::vector<int32_t> seen(comm.size(), -1);
    int32_t next = 0;
    for (int32_t i = 0; i < n0; ++i) {
        const int32_t c = comm[node_of[i]];
        if (seen[c] < 0) seen[c] = next++;
        labels[i] = seen[c];
    }
    return next;
}

// Modularity of token labels (level-0 nodes) at resolution num/den.
double quality(const Graph &g, const int32_t *lab, i64 gnum, i64 gden) {
    std::vector<int32_t> k = degrees(g);
    i64 two_m = 0;
    for (int32_t x : k) two_m += x;
    if (two_m == 0) return 0.0;
    std::vector<i64> E(g.n, 0), K(g.n, 0);
    for (int32_t v = 0; v < g.n; ++v) {
        K[lab[v]] += k[v];
        for (i64 e = g.off[v]; e < g.off[v + 1]; ++e)
            if (lab[g.nbr[e]] == lab[v]) E[lab[v]] += g.w[e];
    }
    __int128 h = 0;
    for (int32_t c = 0; c < g.n; ++c)
        h += __int128(E[c]) * two_m * gden - __int128(gnum) * K[c] * K[c];
    const __int128 den = __int128(two_m) * two_m * gden;
    return double((long double)h / (long double)den);
}

// Largest graph size for which every integer product above stays below 2^62:
// (2m)^2 * max(num, den) * 4.
i64 total_weight(const Graph &g) {
    i64 t = 0;
    for (int32_t x : g.w) t += x;
    return t;
}

bool fits(i64 two_m, i64 gnum, i64 gden) {
    const __int128 m = std::max<i64>(std::max(gnum, gden), 1);
    return __int128(two_m) * two_m * m * 4 < (__int128(1) << 62);
}

template <class F>
void for_each_graph(int32_t G, int32_t n_threads, F &&fn) {
    int32_t t = n_threads > 0 ? n_threads : int32_t(std::thread::hardware_concurrency());
    t = std::max(1, std::min(t, G));
    std::atomic<int32_t> next{0};
    auto work = [&]() {
        for (int32_t g; (g = next.fetch_add(1)) < G;) fn(g);
    };
    std::vector<std::thread> pool;
    for (int32_t i = 1; i < t; ++i) pool.emplace_back(work);
    work();
    for (auto &th : pool) th.join();
}

bool check_args(int32_t G, const int32_t *n_tokens, int32_t n_sinks, const int32_t *edges, int64_t stride,
                int32_t kappa, int64_t gnum, int64_t gden) {
    if (G < 0 || n_sinks < 0 || kappa < 1 || kappa > CKV_MAX_KAPPA || gnum < 0 || gden <= 0) return false;
    if (G > 0 && (!n_tokens || !edges)) return false;
    for (int32_t g = 0; g < G; ++g)
        if (n_tokens[g] < 0 || n_tokens[g] > stride) return false;
    return true;
}

}  // namespace

extern "C" ckv_status ckv_leiden_partition(int32_t n_graphs, const int32_t *n_tokens, int32_t n_sinks,
                                           const int32_t *edges, int64_t row_stride, int32_t kappa,
                                           int64_t gamma_num, int64_t gamma_den, int32_t n_threads,
                                           int32_t *labels, int32_t *n_comm, double *quality_out) {
    if (!check_args(n_graphs, n_tokens, n_sinks, edges, row_stride, kappa, gamma_num, gamma_den))
        return CKV_E_INVALID;
    if (n_graphs > 0 && (!labels || !n_comm)) return CKV_E_INVALID;
    std::vector<ckv_status> st(size_t(std::max(n_graphs, 0)), CKV_OK);
    for_each_graph(n_graphs, n_threads, [&](int32_t g) {
        const int32_t *rows = edges + size_t(g) * size_t(row_stride) * size_t(kappa);
        int32_t *lab = labels + size_t(g) * size_t(row_stride);
        Graph gr;
        if (!token_graph(rows, kappa, n_tokens[g], n_sinks, gr) || !fits(total_weight(gr), gamma_num, gamma_den)) {
            st[g] = CKV_E_INVALID;
            return;
        }
        const int32_t ns = std::min(n_sinks, n_tokens[g]);
        for (int32_t i = 0; i < ns; ++i) lab[i] = -1;
        for (int64_t i = n_tokens[g]; i < row_stride; ++i) lab[i] = -1;
        n_comm[g] = leiden(gr, gamma_num, gamma_den, lab + ns);
        if (quality_out) quality_out[g] = quality(gr, lab + ns, gamma_num, gamma_den);
    });
    for (ckv_status s : st)
        if (s != CKV_OK) return s;
    return CKV_OK;
}

extern "C" ckv_status ckv_partition_quality(int32_t n_graphs, const int32_t *n_tokens, int32_t n_sinks,
                                            const int32_t *edges, int64_t row_stride, int32_t kappa,
                                            int64_t gamma_num, int64_t gamma_den, int32_t n_threads,
                                            const int32_t *labels, double *quality_out) {
    if (!check_args(n_graphs, n_tokens, n_sinks, edges, row_stride, kappa, gamma_num, gamma_den))
        return CKV_E_INVALID;
    if (n_graphs > 0 && (!labels || !quality_out)) return CKV_E_INVALID;
    std::vector<ckv_status> st(size_t(std::max(n_graphs, 0)), CKV_OK);
    for_each_graph(n_graphs, n_threads, [&](int32_t g) {
        const int32_t *rows = edges + size_t(g) * size_t(row_stride) * size_t(kappa);
        const int32_t *lab = labels + size_t(g) * size_t(row_stride);
        Graph gr;
        if (!token_graph(rows, kappa, n_tokens[g], n_sinks, gr) || !fits(total_weight(gr), gamma_num, gamma_den)) {
            st[g] = CKV_E_INVALID;
            return;
        }
        const int32_t ns = std::min(n_sinks, n_tokens[g]);
        for (int32_t i = ns; i < n_tokens[g]; ++i)
            if (lab[i] < 0 || lab[i] >= n_tokens[g] - ns) {
                st[g] = CKV_E_INVALID;
                return;
            }
        quality_out[g] = quality(gr, lab + ns, gamma_num, gamma_den);
    });
    for (ckv_status s : st)
        if (s != CKV_OK) return s;
    return CKV_OK;
}

// Tokens first[g] .. n_tokens[g]-1, in order, join the partition of the tokens
// before them by the vote of their edges (the most common community among the
// labelled targets, ties to the lower id); a token with no labelled target
// starts a community of its own.  Figure 4 runs the partitioning beside the
// model, so the tokens decoded meanwhile are placed by the rule of Figure 1
// panel (3).
extern "C" ckv_status ckv_extend_partition(int32_t n_graphs, const int32_t *first, const int32_t *n_tokens,
                                           const int32_t *edges, int64_t row_stride, int32_t kappa,
                                           int32_t *labels, int32_t *n_comm) {
    if (n_graphs < 0 || kappa < 1 || kappa > CKV_MAX_KAPPA) return CKV_E_INVALID;
    if (n_graphs > 0 && (!first || !n_tokens || !edges || !labels || !n_comm)) return CKV_E_INVALID;
    for (int32_t g = 0; g < n_graphs; ++g)
        if (first[g] < 0 || first[g] > n_tokens[g] || n_tokens[g] > row_stride || n_comm[g] < 0) return CKV_E_INVALID;
    for (int32_t g = 0; g < n_graphs; ++g) {
        const int32_t *rows = edges + size_t(g) * size_t(row_stride) * size_t(kappa);
        for (int32_t i = first[g]; i < n_tokens[g]; ++i)
            for (int32_t e = 0; e < kappa; ++e) {
                const int32_t j = rows[size_t(i) * kappa + e];
                if (j >= i) return CKV_E_INVALID;  // edges point to earlier tokens
            }
    }
    for (int32_t g = 0; g < n_graphs; ++g) {
        const int32_t *rows = edges + size_t(g) * size_t(row_stride) * size_t(kappa);
        int32_t *lab = labels + size_t(g) * size_t(row_stride);
        int32_t c_n = n_comm[g];
        int32_t cand[CKV_MAX_KAPPA], cnt[CKV_MAX_KAPPA];
        for (int32_t i = first[g]; i < n_tokens[g]; ++i) {
            int32_t m = 0;
            for (int32_t e = 0; e < kappa; ++e) {
                const int32_t j = rows[size_t(i) * kappa + e];
                if (j < 0 || lab[j] < 0) continue;
                int32_t k = 0;
                while (k < m && cand[k] != lab[j]) ++k;
                if (k == m) {
                    cand[m] = lab[j];
                    cnt[m++] = 0;
                }
                cnt[k]++;
            }
            if (m == 0) {
                lab[i] = c_n++;
                continue;
            }
            int32_t best = 0;
            for (int32_t k = 1; k < m; ++k)
                if (cnt[k] > cnt[best] || (cnt[k] == cnt[best] && cand[k] < cand[best])) best = k;
            lab[i] = cand[best];
        }
        n_comm[g] = c_n;
    }
    return CKV_OK;
}
