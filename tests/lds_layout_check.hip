// Host-side check of the LDS ring's tile layout, built from the kernel's own
// __host__ __device__ helpers (no GPU needed):
//   * the wave-wide copies of one stage fill every 16-byte slot of the K and V
//     images exactly once and stay inside the stage;
//   * slot (r, c') receives chunk c' ^ swz(r) of key row r (the permutation);
//   * the K fragment reads and the transposing V reads of the MFMA feeds,
//     taken at the reader offsets, see exactly the elements the unpermuted
//     layout would hold at those fragment positions;
//   * reads that the LDS serves together touch distinct banks;
//   * the scalar-base lane offsets equal the per-lane slot addresses;
//   * the 16-row decode engine's transposing V reads deliver V in the key
//     order of the scores each lane holds, on distinct banks;
//   * the stream-K partition names each tile's worker, and its partial slots
//     are unique and inside the workspace.
// Exit status 0 when all hold; the counts of violations are printed.
#include "ua_attn_impl.h"

#include <cstdio>
#include <vector>

using namespace ua;

namespace {

constexpr unsigned kSlotBytes = 4096;  // an arbitrary cache slot stride

template <int D>
int check_layout() {
    typedef LdsGeom<D> L;
    const int img = L::BN * L::RB;  // bytes of one K or V image
    const int slots = 2 * img / 16;
    std::vector<int> writes(slots, 0), src_row(slots, -1), src_chunk(slots, -1);
    int bad = 0;
    for (int w = 0; w < 4; ++w)
        for (int lane = 0; lane < 64; ++lane) {
            LdsCopy<D> cp;
            cp.init(w, lane, kSlotBytes);
            for (int g = 0; g < L::GROUPS; ++g) {
                const int first = (w + 4 * g) * L::ROWS_PER_OP;
                for (int v = 0; v < 2; ++v) {
                    const int byte = (w + 4 * g) * 1024 + v * img + 16 * lane;
                    const int off = v ? cp.voff(g) : cp.koff(g);
                    const unsigned rel = v ? cp.vrel(g) : cp.krel(g);
                    if (byte < 0 || byte + 16 > 2 * img) { ++bad; continue; }
                    if (cp.row(g) < 0 || cp.row(g) >= L::BN || off < 0 || off + 16 > L::RB) ++bad;
                    if (rel != (unsigned)(cp.row(g) - first) * kSlotBytes + (unsigned)off) ++bad;
                    if (cp.row(g) - first < 0 || cp.row(g) - first >= L::ROWS_PER_OP) ++bad;
                    const int slot = byte / 16;
                    ++writes[slot];
                    src_row[slot] = cp.row(g);
                    src_chunk[slot] = off / 16;
                }
            }
        }
    for (int i = 0; i < slots; ++i) {
        if (writes[i] != 1) ++bad;
        const int v = i >= img / 16;
        const int b = (i % (img / 16)) * 16;
        const int r = b / L::RB, cs = (b % L::RB) / 16;
        if (src_row[i] != r) ++bad;
        if (src_chunk[i] != (cs ^ (v ? swz_v<D>(r) : swz_k<D>(r)))) ++bad;
    }
    // (row, column) of the unpermuted tile held at element e of image v
    auto held = [&](int v, int e, int* row, int* col) {
        const int slot = v * img / 16 + (2 * e) / 16;
        *row = src_row[slot];
        *col = src_chunk[slot] * 8 + ((2 * e) % 16) / 2;
    };
    int k_conf = 0, v_conf = 0;
    for (int kt = 0; kt < L::BN / 32; ++kt)
        for (int kc = 0; kc < D / 16; ++kc) {
            // 16-byte reads: 8 lanes per LDS cycle
            std::vector<int> bank(8 * 64, 0);
            for (int lane = 0; lane < 64; ++lane) {
                const Frag f = swizzled_frag<D>(lane);
                // the kernel's expression (lane base per kc & 7, the rest immediate)
                const int off = f.k + kt * 32 * D + 128 * (kc >> 3) + 8 * ((2 * (kc & 7)) ^ f.kx);
                for (int j = 0; j < 8; ++j) {
                    int r, c;
                    held(0, off + j, &r, &c);
                    if (r != 32 * kt + (lane & 31) || c != 16 * kc + 8 * (lane >> 5) + j) ++bad;
                }
                for (int q = 0; q < 4; ++q) ++bank[(lane / 8) * 64 + ((2 * off) / 4 + q) % 64];
            }
            for (int x : bank) k_conf += x > 1;
        }
    for (int kc = 0; kc < L::BN / 16; ++kc)
        for (int dt = 0; dt < D / 32; ++dt)
            for (int hi = 0; hi < 2; ++hi) {
                // 8-byte reads: 16 lanes per LDS cycle
                std::vector<int> bank(4 * 64, 0);
                for (int lane = 0; lane < 64; ++lane) {
                    const Frag f = swizzled_frag<D>(lane);
                    const int off =
                        f.v + kc * 16 * D + 128 * (dt >> 2) + 32 * ((dt & 3) ^ f.vx) + 8 * hi * D;
                    const int g16 = lane >> 4;
                    const int row = 4 * (g16 >> 1) + ((lane & 15) >> 2) + 16 * kc + 8 * hi;
                    const int col = 32 * dt + 16 * (g16 & 1) + 4 * (lane & 3);
                    if ((2 * off) % 8 != 0 || (2 * off) % 16 + 8 > 16) ++bad;
                    for (int j = 0; j < 4; ++j) {
                        int r, c;
                        held(1, off + j, &r, &c);
                        if (r != row || c != col + j) ++bad;
                    }
                    for (int q = 0; q < 2; ++q) ++bank[(lane / 16) * 64 + ((2 * off) / 4 + q) % 64];
                }
                for (int x : bank) v_conf += x > 1;
            }
    std::printf("d=%3d: copies/wave %d, stage %u B: layout violations %d, K bank overlaps %d, "
                "V bank overlaps %d\n",
                D, L::OPS_W, L::STAGE_BYTES, bad, k_conf, v_conf);
    return bad + k_conf + v_conf;
}

// The 16-row decode engine's transposing V reads: lane L of a 16-lane group G
// reads 4 elements at v16_frag_offset(L) (+16 d per block, +16 rows for the
// second read); after the hardware transpose, out(16G + 4a + b)[j] =
// in(16G + 4j + a)[b], lane l must hold V[pi(8 (l / 16) + j)][16 db + l % 16]
// with pi(8g + j) = 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4), the key order of
// the scores the lane holds.
template <int D>
int check_v16() {
    const int vstr = D + kVPad16;
    int bad = 0, conf = 0;
    auto elem = [&](int off, int* row, int* col) { *row = off / vstr; *col = off % vstr; };
    for (int db = 0; db < D / 16; ++db)
        for (int h = 0; h < 2; ++h) {
            int in_row[64][4], in_col[64][4];
            std::vector<int> bank(4 * 64, 0);
            for (int L = 0; L < 64; ++L) {
                const int off = v16_frag_offset<D>(L) + 16 * db + h * 16 * vstr;
                if ((2 * off) % 8) ++bad;
                for (int b = 0; b < 4; ++b) elem(off + b, &in_row[L][b], &in_col[L][b]);
                for (int q = 0; q < 2; ++q) ++bank[(L / 16) * 64 + ((2 * off) / 4 + q) % 64];
            }
            for (int x : bank) conf += x > 1;
            for (int l = 0; l < 64; ++l) {
                const int G = l / 16, a = (l % 16) / 4, b = l % 4;
                for (int j = 0; j < 4; ++j) {
                    const int src = 16 * G + 4 * j + a;
                    const int key = (h ? 16 : 0) + 4 * G + j;  // pi(8G + 4h + j)
                    if (in_row[src][b] != key || in_col[src][b] != 16 * db + l % 16) ++bad;
                }
            }
        }
    std::printf("d=%3d (16-row V reads): violations %d, bank overlaps %d\n", D, bad, conf);
    return bad + conf;
}

// The stream-K partition: W workers split T flattened tiles into contiguous
// ranges [jT/W, (j+1)T/W); sk_worker_of(x) must name the worker holding tile
// x; and with random per-unit tile counts the partial slots (u + j) * H + w of
// every (unit u, worker j) a worker touches, for each of the H waves w of a
// worker (the kv heads of one head group), are unique and below
// (number of units + W) * H, and the reduce's walk from the unit's first
// worker with stride H meets exactly those slots.  (N and G below are the
// unit and worker counts.)
int check_stream_k() {
    int bad = 0;
    unsigned rng = 12345u;
    auto next = [&]() { rng = rng * 1664525u + 1013904223u; return rng >> 8; };
    for (int trial = 0; trial < 400; ++trial) {
        const int N = 1 + next() % 70;
        std::vector<int> n(N);
        int64_t T = 0;
        for (int s = 0; s < N; ++s) {
            n[s] = next() % 5 == 0 ? 0 : (int)(next() % 300);
            T += n[s];
        }
        const int64_t G = 1 + next() % 2100;
        if (T == 0) continue;
        std::vector<int> first(N + 1, 0);
        for (int s = 0; s < N; ++s) first[s + 1] = first[s] + n[s];
        const int H = 1 << (trial % 4);  // waves per worker: 1, 2, 4, 8
        std::vector<char> used((size_t)(N + G) * H, 0);
        for (int64_t g = 0; g < G; ++g) {
            const int64_t A = g * T / G, B = (g + 1) * T / G;
            for (int64_t x = A; x < B; ++x)
                if (sk_worker_of(x, T, G) != g) ++bad;
            if (A >= B) continue;
            // units the worker touches: those whose tile range meets [A, B)
            for (int s = 0; s < N; ++s) {
                if (n[s] == 0 || first[s + 1] <= A || first[s] >= B) continue;
                for (int w = 0; w < H; ++w) {
                    const int64_t slot = (s + g) * H + w;
                    if (slot >= (N + G) * H || used[slot]) ++bad;
                    used[slot] = 1;
                }
            }
        }
        // the reduce reads slot ((s + g0) * H + w) + k * H for k = 0 .. g1 - g0
        for (int s = 0; s < N; ++s) {
            if (n[s] == 0) continue;
            const int g0 = sk_worker_of(first[s], T, G), g1 = sk_worker_of(first[s] + n[s] - 1, T, G);
            for (int w = 0; w < H; ++w)
                for (int g = g0; g <= g1; ++g) {
                    const int64_t A = (int64_t)g * T / G, B = (int64_t)(g + 1) * T / G;
                    const int64_t slot = ((int64_t)(s + g0) * H + w) + (int64_t)(g - g0) * H;
                    if (A < B && (slot >= (N + G) * H || !used[slot])) ++bad;
                }
        }
        // a sequence's groups: from the group of its first tile to that of its last
        for (int s = 0; s < N; ++s) {
            if (n[s] == 0) continue;
            const int g0 = sk_worker_of(first[s], T, G), g1 = sk_worker_of(first[s] + n[s] - 1, T, G);
            for (int g = g0; g <= g1; ++g) {
                const int64_t A = (int64_t)g * T / G, B = (int64_t)(g + 1) * T / G;
                const bool live = A < B;
                const bool meets = A < B && first[s + 1] > A && first[s] < B;
                if (live != meets) ++bad;
            }
        }
    }
    std::printf("stream-K partition: violations %d\n", bad);
    return bad;
}

}  // namespace

int main() {
    const int bad = check_layout<64>() + check_layout<128>() + check_layout<256>() +
                    check_v16<64>() + check_v16<128>() + check_v16<256>() + check_stream_k();
    std::printf(bad ? "FAIL\n" : "OK\n");
    return bad != 0;
}
