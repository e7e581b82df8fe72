// Host-side check of the LDS ring's tile layout, built from the kernel's own
// __host__ __device__ helpers (no GPU needed):
//   * the wave-wide copies of one stage fill every 16-byte slot of the K and V
//     images exactly once and stay inside the stage;
//   * slot (r, c') receives chunk c' ^ swz(r) of key row r (the permutation);
//   * the K fragment reads and the transposing V reads of the MFMA feeds,
//     taken at the reader offsets, see exactly the elements the unpermuted
//     layout would hold at those fragment positions;
//   * reads that the LDS serves together touch distinct banks;
//   * the scalar-base lane offsets equal the per-lane slot addresses.
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
                    const int off = v ? cp.voff[g] : cp.koff[g];
                    const unsigned rel = v ? cp.vrel[g] : cp.krel[g];
                    if (byte < 0 || byte + 16 > 2 * img) { ++bad; continue; }
                    if (cp.row[g] < 0 || cp.row[g] >= L::BN || off < 0 || off + 16 > L::RB) ++bad;
                    if (rel != (unsigned)(cp.row[g] - first) * kSlotBytes + (unsigned)off) ++bad;
                    if (cp.row[g] - first < 0 || cp.row[g] - first >= L::ROWS_PER_OP) ++bad;
                    const int slot = byte / 16;
                    ++writes[slot];
                    src_row[slot] = cp.row[g];
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
                const int off = f.k + kt * 32 * D + 8 * ((2 * kc) ^ f.kx);
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
                    const int off = f.v + kc * 16 * D + 32 * (dt ^ f.vx) + 8 * hi * D;
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

}  // namespace

int main() {
    const int bad = check_layout<64>() + check_layout<128>() + check_layout<256>();
    std::printf(bad ? "FAIL\n" : "OK\n");
    return bad != 0;
}
