// Host calibration of the transform-coded KV cache: statistics, Jacobi KLT, attention-aware
// channel weights, reverse water-filling and exact-budget integer bits, Gaussian-optimal
// uniform quantizer steps, codebook construction, persistence and the per-head device blob.
//
// Method references (pages): "Attention-Aware Transform Coding Guide", sections
// "Decorrelation via the Karhunen-Loeve Transform (KLT)" (covariances, eigenbasis),
// "Theorem: Additive Error Decomposition" (key/value weights) and "Optimal Bit Allocation
// via Reverse Water-Filling" (R_j = max(0, 1/2 log2(w_j lambda_j / theta)), sum R_j fixed);
// "KV Cache Compression Through the Lens of Transform Coding", Methodology (whitening).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <thread>

#include "aatc_internal.h"

namespace aatc {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

uint16_t f32_to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Run fn(i) for i in [0, n) on up to hardware_concurrency threads.
template <class F>
static void parallel_for(int64_t n, F fn) {
    unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    if (n < 2 || nt == 1) {
        for (int64_t i = 0; i < n; ++i) fn(i, 0u);
        return;
    }
    nt = (unsigned)std::min<int64_t>(nt, n);
    std::atomic<int64_t> next(0);
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            for (int64_t i; (i = next.fetch_add(1)) < n;) fn(i, t);
        });
    for (auto& x : th) x.join();
}

static unsigned n_workers() {
    return std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
}

// ------------------------------------------------------------------------------------
// Symmetric eigensolver: cyclic Jacobi rotations (fp64), eigenvalues descending, each
// eigenvector's largest-magnitude entry positive (lowest row index on ties).
// ------------------------------------------------------------------------------------
static int jacobi_eigen(int d, const double* S, int max_sweeps, std::vector<double>& lam,
                        std::vector<double>& U) {
    std::vector<double> A(S, S + (size_t)d * d), Vm((size_t)d * d, 0.0);
    for (int i = 0; i < d; ++i) Vm[(size_t)i * d + i] = 1.0;
    double fro = 0.0;
    for (size_t i = 0; i < A.size(); ++i) fro += A[i] * A[i];
    fro = std::sqrt(fro);
    bool converged = fro == 0.0;
    for (int sweep = 0; sweep < max_sweeps && !converged; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < d; ++p)
            for (int q = p + 1; q < d; ++q) off += A[(size_t)p * d + q] * A[(size_t)p * d + q];
        if (std::sqrt(2.0 * off) <= 1e-15 * fro) {
            converged = true;
            break;
        }
        for (int p = 0; p < d - 1; ++p) {
            for (int q = p + 1; q < d; ++q) {
                double apq = A[(size_t)p * d + q];
                if (apq == 0.0) continue;
                double app = A[(size_t)p * d + p], aqq = A[(size_t)q * d + q];
                double th = (aqq - app) / (2.0 * apq);
                double t = (th >= 0 ? 1.0 : -1.0) / (std::fabs(th) + std::sqrt(th * th + 1.0));
                double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
                for (int k = 0; k < d; ++k) {  // columns p, q
                    double akp = A[(size_t)k * d + p], akq = A[(size_t)k * d + q];
                    A[(size_t)k * d + p] = c * akp - s * akq;
                    A[(size_t)k * d + q] = s * akp + c * akq;
                }
                for (int k = 0; k < d; ++k) {  // rows p, q
                    double apk = A[(size_t)p * d + k], aqk = A[(size_t)q * d + k];
                    A[(size_t)p * d + k] = c * apk - s * aqk;
                    A[(size_t)q * d + k] = s * apk + c * aqk;
                }
                A[(size_t)p * d + q] = A[(size_t)q * d + p] = 0.0;
                for (int k = 0; k < d; ++k) {
                    double vkp = Vm[(size_t)k * d + p], vkq = Vm[(size_t)k * d + q];
                    Vm[(size_t)k * d + p] = c * vkp - s * vkq;
                    Vm[(size_t)k * d + q] = s * vkp + c * vkq;
                }
            }
        }
    }
    if (!converged) {
        double off = 0.0;
        for (int p = 0; p < d; ++p)
            for (int q = p + 1; q < d; ++q) off += A[(size_t)p * d + q] * A[(size_t)p * d + q];
        if (!(std::sqrt(2.0 * off) <= 1e-15 * fro))
            return set_error(AATC_ERR_NO_CONVERGENCE, "Jacobi eigensolver did not converge in %d sweeps",
                             max_sweeps);
    }
    std::vector<int> order(d);
    for (int i = 0; i < d; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        return A[(size_t)a * d + a] > A[(size_t)b * d + b];
    });
    lam.assign(d, 0.0);
    U.assign((size_t)d * d, 0.0);
    for (int j = 0; j < d; ++j) {
        int o = order[j];
        lam[j] = std::max(0.0, A[(size_t)o * d + o]);
        int imax = 0;
        double vmax = -1.0;
        for (int i = 0; i < d; ++i) {
            double v = std::fabs(Vm[(size_t)i * d + o]);
            if (v > vmax) {
                vmax = v;
                imax = i;
            }
        }
        double sgn = Vm[(size_t)imax * d + o] < 0 ? -1.0 : 1.0;
        for (int i = 0; i < d; ++i) U[(size_t)i * d + j] = sgn * Vm[(size_t)i * d + o];
    }
    return AATC_OK;
}

// ------------------------------------------------------------------------------------
// Reverse water-filling (continuous), for reporting the water level theta.
// ------------------------------------------------------------------------------------
static double waterfill_theta(const std::vector<double>& x, double total, int max_bits) {
    double xmin = INFINITY, xmax = 0.0;
    int npos = 0;
    for (double v : x)
        if (v > 0) {
            xmin = std::min(xmin, v);
            xmax = std::max(xmax, v);
            ++npos;
        }
    if (total <= 0 || npos == 0) return INFINITY;
    if (total >= (double)max_bits * npos) return 0.0;
    auto rate = [&](double lt) {
        double s = 0.0;
        for (double v : x)
            if (v > 0) {
                double r = 0.5 * (std::log2(v) - lt / std::log(2.0));
                s += std::min<double>(std::max(r, 0.0), max_bits);
            }
        return s;
    };
    double lo = std::log(xmin) - 2.0 * max_bits * std::log(2.0) - 1.0, hi = std::log(xmax);
    for (int it = 0; it < 400; ++it) {
        double mid = 0.5 * (lo + hi);
        if (rate(mid) > total)
            lo = mid;
        else
            hi = mid;
        if (hi - lo < 1e-15 * std::max(1.0, std::fabs(mid))) break;
    }
    return std::exp(0.5 * (lo + hi));
}

// Exact-budget integer allocation of one group of channels: the `budget` largest marginal
// gains x_j 4^-k (k < max_bits), ties broken by lower channel then lower k.
static std::vector<int32_t> greedy_bits(const std::vector<double>& x, int budget, int max_bits) {
    struct Gain {
        double g;
        int j, k;
    };
    std::vector<Gain> c;
    for (int j = 0; j < (int)x.size(); ++j)
        for (int k = 0; k < max_bits; ++k) c.push_back({std::ldexp(x[j], -2 * k), j, k});
    std::sort(c.begin(), c.end(), [](const Gain& a, const Gain& b) {
        if (a.g != b.g) return a.g > b.g;
        if (a.j != b.j) return a.j < b.j;
        return a.k < b.k;
    });
    std::vector<int32_t> bits(x.size(), 0);
    for (int i = 0; i < budget && i < (int)c.size(); ++i) bits[c[i].j] += 1;
    return bits;
}

static double alloc_cost(const std::vector<double>& x, const std::vector<int32_t>& b) {
    double s = 0.0;
    for (size_t j = 0; j < x.size(); ++j) s += std::ldexp(x[j], -2 * b[j]);
    return s;
}

// Joint allocation with the keys' total a multiple of key_align bits (whole record words):
// every admissible key budget is solved exactly for keys and values, the cheapest split
// wins (ties: smaller key budget).
static void allocate_joint(const std::vector<double>& xK, const std::vector<double>& xV, int total, int max_bits,
                           int key_align, std::vector<int32_t>& bK, std::vector<int32_t>& bV) {
    const int d = (int)xK.size();
    double best = INFINITY;
    for (int bk = 0; bk <= std::min(total, d * max_bits); bk += key_align) {
        const int bv = total - bk;
        if (bv > d * max_bits) continue;
        std::vector<int32_t> k = greedy_bits(xK, bk, max_bits), v = greedy_bits(xV, bv, max_bits);
        const double cost = alloc_cost(xK, k) + alloc_cost(xV, v);
        if (cost < best) {
            best = cost;
            bK = k;
            bV = v;
        }
    }
}

// ------------------------------------------------------------------------------------
// Gaussian-optimal midrise uniform quantizer (unit variance, 2^b levels): root of the
// MSE's derivative with respect to the step (reconstruction points move, cell boundaries
// contribute nothing to first order).
// ------------------------------------------------------------------------------------
static double phi(double x) { return std::isfinite(x) ? std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI) : 0.0; }
static double Phi(double x) {
    if (x == INFINITY) return 1.0;
    if (x == -INFINITY) return 0.0;
    return 0.5 * std::erfc(-x / std::sqrt(2.0));
}

static double mse_slope(double step, int levels) {
    int half = levels / 2;
    double total = 0.0;
    for (int k = -half; k < half; ++k) {
        double a = k == -half ? -INFINITY : k * step;
        double b = k == half - 1 ? INFINITY : (k + 1) * step;
        double c = k + 0.5;
        total += c * (c * step * (Phi(b) - Phi(a)) - (phi(a) - phi(b)));
    }
    return total;
}

static double optimal_step(int bits) {
    int levels = 1 << bits;
    double lo = 1e-4, hi = 4.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mse_slope(mid, levels) < 0.0)
            lo = mid;
        else
            hi = mid;
        if (hi - lo <= 4e-16 * hi) break;
    }
    return 0.5 * (lo + hi);
}

static const double* step_table() {
    static double tab[9];
    static bool init = false;
    if (!init) {
        tab[0] = 0.0;
        for (int b = 1; b <= 8; ++b) tab[b] = optimal_step(b);
        init = true;
    }
    return tab;
}

// ------------------------------------------------------------------------------------
// derived tables and device blob
// ------------------------------------------------------------------------------------
// Byte-aligned fields of one record (the packed layout): channels with b > 0, widest
// first (ties: lower channel), each whole in the lowest-index byte with room, at that
// byte's lowest free bit; channels left over are cut into pieces that fill free bits byte
// by byte (lowest code bits first); finally bytes are renumbered by decreasing field
// count (ties: lower byte).  Returns false if the bits do not fill whole bytes.
static bool make_fields(const std::vector<int32_t>& bits, std::vector<Field>& out, int& total) {
    out.clear();
    total = 0;
    for (int b : bits) total += b;
    if (total % 8) return false;
    const int nbytes = total / 8;
    std::vector<int> free(nbytes, 8), order, left;
    for (int j = 0; j < (int)bits.size(); ++j)
        if (bits[j] > 0) order.push_back(j);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return bits[a] > bits[b]; });
    for (int j : order) {
        int q = 0;
        while (q < nbytes && free[q] < bits[j]) ++q;
        if (q == nbytes) {
            left.push_back(j);
            continue;
        }
        out.push_back({j, bits[j], 0, q, 8 - free[q]});
        free[q] -= bits[j];
    }
    for (int j : left) {
        int e = 0;
        for (int q = 0; q < nbytes && e < bits[j]; ++q) {
            const int w = std::min(free[q], bits[j] - e);
            if (w <= 0) continue;
            out.push_back({j, w, e, q, 8 - free[q]});
            free[q] -= w;
            e += w;
        }
    }
    std::vector<int> count(nbytes, 0), byrank(nbytes), rank(nbytes);
    for (const Field& f : out) ++count[f.byte];
    for (int q = 0; q < nbytes; ++q) byrank[q] = q;
    std::stable_sort(byrank.begin(), byrank.end(), [&](int a, int b) { return count[a] > count[b]; });
    for (int i = 0; i < nbytes; ++i) rank[byrank[i]] = i;
    for (Field& f : out) f.byte = rank[f.byte];
    std::sort(out.begin(), out.end(),
              [](const Field& a, const Field& b) { return a.byte != b.byte ? a.byte < b.byte : a.pos < b.pos; });
    return true;
}

// Decode schedule of one head (see DevHead).  Scores: every key-record word is split
// into "dwords", one per field index within a byte; each dword keeps one field per byte
// under a mask.  Dwords fill the score MFMAs in record order, 16 per MFMA (four per lane
// group).  Values: one MFMA column per value field, 16 per column block.
static int build_decode_schedule(const HeadCB& H, DevHead& D) {
    for (int m = 0; m < kMaxQM; ++m)
        for (int g = 0; g < 4; ++g) {
            for (int i = 0; i < 8; ++i) D.kq_sched[m][g][i] = 0u;
            for (int i = 0; i < 16; ++i) D.kq_slot[m][g][i] = 0xFFFF;
        }
    struct Dword {
        int word;
        uint32_t mask;
        uint16_t slot[4];
    };
    std::vector<Dword> dws;
    const int WK = H.BK / 32;
    for (int r = 0; r < WK; ++r) {
        std::vector<const Field*> fb[4];
        for (const Field& f : H.fK)
            if (f.byte / 4 == r) fb[f.byte % 4].push_back(&f);  // in bit order (fields are sorted)
        size_t nd = 0;
        for (int b = 0; b < 4; ++b) nd = std::max(nd, fb[b].size());
        for (size_t j = 0; j < nd; ++j) {
            Dword dw{r, 0u, {0xFFFF, 0xFFFF, 0xFFFF, 0xFFFF}};
            for (int b = 0; b < 4; ++b) {
                if (j >= fb[b].size()) continue;
                const Field& f = *fb[b][j];
                dw.mask |= ((1u << f.width) - 1u) << (8 * b + f.pos);
                const int flip = f.pos + f.width == 8 ? 1 : 0;
                dw.slot[b] = (uint16_t)(f.chan | (f.shift << 8) | (f.pos << 11) | (flip << 14));
            }
            dws.push_back(dw);
        }
    }
    const int nqm = ((int)dws.size() + 15) / 16;
    if (nqm > kMaxQM) return AATC_ERR_UNSUPPORTED;
    D.nqm = std::max(nqm, 1);
    for (size_t k = 0; k < dws.size(); ++k) {
        const int m = (int)k / 16, g = ((int)k / 4) % 4, i = (int)k % 4;
        D.kq_sched[m][g][i] = 256u * (uint32_t)dws[k].word;
        D.kq_sched[m][g][4 + i] = dws[k].mask;
        for (int b = 0; b < 4; ++b) D.kq_slot[m][g][4 * i + b] = dws[k].slot[b];
    }
    for (int j = 0; j < kMaxD; ++j) D.kq_fmax[j] = 0.0f;
    for (const Field& f : H.fK) D.kq_fmax[f.chan] = std::max(D.kq_fmax[f.chan], std::ldexp(1.0f, f.shift - f.pos));
    // value columns
    const int nf = (int)H.fV.size();
    D.nvb = std::max((nf + 15) / 16, 1);
    if (D.nvb > kMaxVB || nf > kMaxFields) return AATC_ERR_UNSUPPORTED;
    for (int cb = 0; cb < kMaxVB; ++cb)
        for (int c = 0; c < 16; ++c) D.vb_col[cb][c] = 0u;
    for (int i = 0; i < nf; ++i) {
        const Field& f = H.fV[i];
        D.vb_col[i / 16][i % 16] = (uint32_t)(64 * f.byte) | ((((1u << f.width) - 1u) << f.pos) << 16);
    }
    for (int j = 0; j < kMaxD; ++j)
        for (int k = 0; k < 8; ++k) D.vch[j][k] = 0xFFFF;
    for (int i = 0; i < nf; ++i) {
        const Field& f = H.fV[i];
        int k = 0;
        while (k < 8 && D.vch[f.chan][k] != 0xFFFF) ++k;
        if (k == 8) return AATC_ERR_UNSUPPORTED;
        const int flip = f.pos + f.width == 8 ? 1 : 0;
        D.vch[f.chan][k] = (uint16_t)(i | ((f.shift - f.pos + 8) << 9) | (flip << 13));
    }
    return AATC_OK;
}

// Channel order of the encoder's MFMA columns (fields by channel in `fs`, sorted by channel
// then shift): 16-column blocks whose channels' first fields sit in record bytes distinct mod
// 16 (the encoder's staged block puts record byte q in LDS bank group q mod 16), filled
// greedily from the largest residue classes; channels without bits fill the rest.
static void build_encoder_order(const std::vector<Field>& fs, int d, uint8_t* perm) {
    std::vector<int> first_byte(d, -1);
    for (const Field& f : fs)
        if (first_byte[f.chan] < 0) first_byte[f.chan] = f.byte;  // fs: by channel, lowest shift first
    std::vector<std::vector<int>> cls(16);
    std::vector<int> uncoded;
    for (int j = 0; j < d; ++j) (first_byte[j] < 0 ? uncoded : cls[first_byte[j] % 16]).push_back(j);
    const int nblk = d / 16;
    std::vector<std::vector<int>> blk(nblk);
    std::vector<uint32_t> used(nblk, 0u);
    std::vector<int> order(16);
    for (int r = 0; r < 16; ++r) order[r] = r;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cls[a].size() > cls[b].size(); });
    std::vector<int> spill;
    for (int r : order)
        for (int j : cls[r]) {
            int best = -1;
            for (int k = 0; k < nblk; ++k)
                if (!(used[k] >> r & 1u) && blk[k].size() < 16 && (best < 0 || blk[k].size() < blk[best].size())) best = k;
            if (best < 0) {
                spill.push_back(j);
                continue;
            }
            blk[best].push_back(j);
            used[best] |= 1u << r;
        }
    for (int j : spill) uncoded.insert(uncoded.begin(), j);
    size_t u = 0;
    for (int k = 0; k < nblk; ++k) {
        while (blk[k].size() < 16 && u < uncoded.size()) blk[k].push_back(uncoded[u++]);
        for (int c = 0; c < 16; ++c) perm[16 * k + c] = (uint8_t)blk[k][c];
    }
}

// Inverse of a d x d matrix (row-major) by Gauss-Jordan elimination with partial pivoting,
// in fp64.  Returns false for a (numerically) singular matrix.
static bool invert(int d, const std::vector<double>& A, std::vector<double>& inv) {
    std::vector<double> M(A);
    inv.assign((size_t)d * d, 0.0);
    for (int i = 0; i < d; ++i) inv[(size_t)i * d + i] = 1.0;
    double scale = 0.0;
    for (double v : A) scale = std::max(scale, std::fabs(v));
    if (!(scale > 0.0) || !std::isfinite(scale)) return false;
    for (int c = 0; c < d; ++c) {
        int piv = c;
        for (int r = c + 1; r < d; ++r)
            if (std::fabs(M[(size_t)r * d + c]) > std::fabs(M[(size_t)piv * d + c])) piv = r;
        const double pv = M[(size_t)piv * d + c];
        if (!(std::fabs(pv) > 1e-13 * scale)) return false;
        if (piv != c)
            for (int k = 0; k < d; ++k) {
                std::swap(M[(size_t)piv * d + k], M[(size_t)c * d + k]);
                std::swap(inv[(size_t)piv * d + k], inv[(size_t)c * d + k]);
            }
        const double ip = 1.0 / pv;
        for (int k = 0; k < d; ++k) {
            M[(size_t)c * d + k] *= ip;
            inv[(size_t)c * d + k] *= ip;
        }
        for (int r = 0; r < d; ++r) {
            if (r == c) continue;
            const double f = M[(size_t)r * d + c];
            if (f == 0.0) continue;
            for (int k = 0; k < d; ++k) {
                M[(size_t)r * d + k] -= f * M[(size_t)c * d + k];
                inv[(size_t)r * d + k] -= f * inv[(size_t)c * d + k];
            }
        }
    }
    for (double v : inv)
        if (!std::isfinite(v)) return false;
    return true;
}

// ------------------------------------------------------------------------------------
// Vector-quantized keys ("Spend Bits Where Queries Look", abstract: equal-volume groups,
// equal-size codebooks).  Groups of kVqDim coefficients: the kVqDim * n_g of largest
// weight (ties: lower channel), formed greedily toward equal volume prod x_j - largest
// weight first, each into the unfilled group with the smallest sum of log(x_j / x_min)
// (ties: lower group).  Output: channels of group g at chan[g * kVqDim ..], ascending.
// ------------------------------------------------------------------------------------
static bool vq_groups(const std::vector<double>& x, int n_g, std::vector<int32_t>& chan) {
    const int d = (int)x.size(), n = kVqDim * n_g;
    std::vector<int> order(d);
    for (int j = 0; j < d; ++j) order[j] = j;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return x[a] > x[b]; });
    order.resize(n);  // coded channels, by decreasing weight (ties: lower index)
    double xmin = x[order[n - 1]];
    if (!(xmin > 0)) return false;
    std::vector<double> load(n_g, 0.0);
    std::vector<std::vector<int32_t>> mem(n_g);
    for (int j : order) {
        int best = -1;
        for (int g = 0; g < n_g; ++g)
            if ((int)mem[g].size() < kVqDim && (best < 0 || load[g] < load[best])) best = g;
        mem[best].push_back(j);
        load[best] += std::log(x[j] / xmin);
    }
    chan.clear();
    for (auto& m : mem) {
        std::sort(m.begin(), m.end());
        chan.insert(chan.end(), m.begin(), m.end());
    }
    return true;
}

// Lloyd's algorithm in fp64 on points y [n][kVqDim]: iters rounds of nearest-word
// assignment (squared distance summed in coordinate order, lowest index on ties) and
// cell means (an empty cell keeps its word); initial words: the first kVqSize points.
static void lloyd(const std::vector<double>& y, int64_t n, int iters, std::vector<double>& code) {
    code.assign(y.begin(), y.begin() + (size_t)kVqSize * kVqDim);
    std::vector<int32_t> a(n);
    std::vector<double> sum((size_t)kVqSize * kVqDim);
    std::vector<int64_t> cnt(kVqSize);
    for (int it = 0; it < iters; ++it) {
        for (int64_t i = 0; i < n; ++i) {
            const double* p = &y[(size_t)i * kVqDim];
            double best = 0.0;
            int bi = 0;
            for (int c = 0; c < kVqSize; ++c) {
                const double* z = &code[(size_t)c * kVqDim];
                double e = 0.0;
                for (int k = 0; k < kVqDim; ++k) e += (p[k] - z[k]) * (p[k] - z[k]);
                if (c == 0 || e < best) best = e, bi = c;
            }
            a[i] = bi;
        }
        std::fill(sum.begin(), sum.end(), 0.0);
        std::fill(cnt.begin(), cnt.end(), 0);
        for (int64_t i = 0; i < n; ++i) {
            ++cnt[a[i]];
            for (int k = 0; k < kVqDim; ++k) sum[(size_t)a[i] * kVqDim + k] += y[(size_t)i * kVqDim + k];
        }
        for (int c = 0; c < kVqSize; ++c)
            if (cnt[c])
                for (int k = 0; k < kVqDim; ++k) code[(size_t)c * kVqDim + k] = sum[(size_t)c * kVqDim + k] / (double)cnt[c];
    }
}

int finalize(aatc_codebook* cb) {
    const int d = cb->d;
    int total = -1;
    for (size_t h = 0; h < cb->heads.size(); ++h) {
        HeadCB& H = cb->heads[h];
        for (int j = 0; j < d; ++j) {
            if (H.bK[j] < 0 || H.bK[j] > 8 || H.bV[j] < 0 || H.bV[j] > 8)
                return set_error(AATC_ERR_BUDGET, "head %zu: bits out of [0,8]", h);
            if ((H.bK[j] > 0 && !(H.stepK[j] > 0 && std::isfinite(H.stepK[j]))) ||
                (H.bV[j] > 0 && !(H.stepV[j] > 0 && std::isfinite(H.stepV[j]))))
                return set_error(AATC_ERR_STATS, "head %zu channel %d: coded channel needs a positive step", h, j);
        }
        if (H.vq_groups) {
            const int n_g = H.vq_groups;
            if (n_g % 4 || kVqDim * n_g > d || (int)H.vq_chan.size() != kVqDim * n_g ||
                (int)H.vq_scale.size() != d || H.vq_cent.size() != (size_t)n_g * kVqSize * kVqDim)
                return set_error(AATC_ERR_BUDGET, "head %zu: vector-quantized keys need a multiple of 4 groups "
                                 "of 4 channels (at most d / 4 groups)", h);
            std::vector<int> seen(d, 0);
            for (int32_t j : H.vq_chan) {
                if (j < 0 || j >= d || seen[j]++)
                    return set_error(AATC_ERR_INVALID_ARG, "head %zu: group channels must be distinct and in [0, d)", h);
                if (!(H.vq_scale[j] > 0 && std::isfinite(H.vq_scale[j])))
                    return set_error(AATC_ERR_INVALID_ARG, "head %zu channel %d: coded channel needs a positive scale", h, j);
            }
            for (float z : H.vq_cent)
                if (!std::isfinite(z)) return set_error(AATC_ERR_INVALID_ARG, "head %zu: non-finite codeword", h);
            for (int j = 0; j < d; ++j)
                if (H.bK[j]) return set_error(AATC_ERR_INVALID_ARG, "head %zu: scalar key bits with vector-quantized keys", h);
        }
        const std::vector<int32_t> keybits = H.vq_groups ? std::vector<int32_t>(H.vq_groups, 8) : H.bK;
        if (!make_fields(keybits, H.fK, H.BK) || !make_fields(H.bV, H.fV, H.BV))
            return set_error(AATC_ERR_BUDGET, "head %zu: key and value bits per token must be whole bytes", h);
        if ((int)H.fK.size() > kMaxFields || (int)H.fV.size() > kMaxFields)
            return set_error(AATC_ERR_UNSUPPORTED, "head %zu: more than %d fields in a record", h, kMaxFields);
        if (H.BK % kKeyAlign)
            return set_error(AATC_ERR_BUDGET, "head %zu: key bits per token (%d) must be a multiple of %d", h, H.BK,
                             kKeyAlign);
        if (H.vq_groups != cb->heads[0].vq_groups)
            return set_error(AATC_ERR_INVALID_ARG, "head %zu: every head of a codebook has the same key quantizer", h);
        int B = H.BK + H.BV;
        if (total < 0) total = B;
        if (B != total) return set_error(AATC_ERR_BUDGET, "head %zu has %d bits per token, head 0 has %d", h, B, total);
    }
    if (total <= 0 || total % 8) return set_error(AATC_ERR_BUDGET, "bits per token (%d) must be a positive multiple of 8", total);
    cb->total_bits = total;

    cb->blob.assign(cb->heads.size(), DevHead());
    for (size_t h = 0; h < cb->heads.size(); ++h) {
        const HeadCB& H = cb->heads[h];
        DevHead& D = cb->blob[h];
        std::memset(&D, 0, sizeof(DevHead));
        D.d = d;
        D.BK = H.BK;
        D.BV = H.BV;
        D.nfK = (int)H.fK.size();
        D.nfV = (int)H.fV.size();
        D.enc_terms = enc_terms_for(cb->total_bits, d);
        for (int which = 0; which < 2; ++which) {
            const std::vector<double>& U = which ? H.UV : H.UK;
            const std::vector<double>& mu = which ? H.muV : H.muK;
            const std::vector<int32_t>& bits = which ? H.bV : H.bK;
            const std::vector<float>& step = which ? H.stepV : H.stepK;
            float* U32 = which ? D.UV : D.UK;
            uint16_t* hi = which ? D.EVt_hi : D.EKt_hi;  // [j * d + i]
            uint16_t* lo = which ? D.EVt_lo : D.EKt_lo;
            uint16_t* mid = which ? D.EVt_mid : D.EKt_mid;
            float* start = which ? D.estartV : D.estartK;
            for (int j = 0; j < d; ++j) {
                // the fp32 reciprocal step of the quantizer (0: uncoded channel)
                const double inv = bits[j] ? (double)(float)(1.0 / (double)step[j]) : 0.0;
                double s = 0.0;
                for (int i = 0; i < d; ++i) {
                    U32[i * d + j] = (float)U[(size_t)i * d + j];
                    const float w = (float)(U[(size_t)i * d + j] * inv);
                    hi[j * d + i] = f32_to_bf16(w);
                    lo[j * d + i] = f32_to_bf16(w - bf16_to_f32(hi[j * d + i]));
                    mid[j * d + i] = D.enc_terms == 3
                                         ? f32_to_bf16(w - bf16_to_f32(hi[j * d + i]) - bf16_to_f32(lo[j * d + i]))
                                         : (uint16_t)0;
                    s += mu[i] * ((double)bf16_to_f32(hi[j * d + i]) + (double)bf16_to_f32(lo[j * d + i]) +
                                  (double)bf16_to_f32(mid[j * d + i]));
                }
                start[j] = bits[j] ? (float)((double)(1 << (bits[j] - 1)) - 0.5 - s) : 0.0f;
            }
        }
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) D.UVt[j * d + i] = D.UV[i * d + j];
        // query transform: coefficients c = (k - mu) T, so q.k = (T^{-1} q).c + q.mu
        std::vector<double> Tinv;
        if (!invert(d, H.UK, Tinv)) return set_error(AATC_ERR_INVALID_ARG, "head %zu: the key basis is not invertible", h);
        for (int j = 0; j < d; ++j)
            for (int i = 0; i < d; ++i) {
                const float u = (float)Tinv[(size_t)j * d + i];
                D.QKt_hi[j * d + i] = f32_to_bf16(u);
                D.QKt_lo[j * d + i] = f32_to_bf16(u - bf16_to_f32(D.QKt_hi[j * d + i]));
            }
        for (int j = 0; j < d; ++j) {
            D.muV[j] = (float)H.muV[j];
            D.muK[j] = (float)H.muK[j];
            D.bitsK[j] = H.bK[j];
            D.bitsV[j] = H.bV[j];
            D.stepK[j] = H.bK[j] ? H.stepK[j] : 0.0f;
            D.stepV[j] = H.bV[j] ? H.stepV[j] : 0.0f;
            D.invK[j] = H.bK[j] ? (float)(1.0 / (double)H.stepK[j]) : 0.0f;
            D.invV[j] = H.bV[j] ? (float)(1.0 / (double)H.stepV[j]) : 0.0f;
        }
        // output offset: the dequantized value coefficient is step (code - 2^(b-1) + 1/2), so
        // o = mu_V + U_V (step * code_mean) - U_V (step * (2^(b-1) - 1/2))
        for (int i = 0; i < d; ++i) {
            double o = H.muV[i];
            for (int j = 0; j < d; ++j)
                if (H.bV[j] > 0) o -= H.UV[(size_t)i * d + j] * (double)H.stepV[j] * ((double)(1 << (H.bV[j] - 1)) - 0.5);
            D.obias[i] = (float)o;
        }
        for (int which = 0; which < 2; ++which) {
            std::vector<Field> fs = which ? H.fV : H.fK;
            std::stable_sort(fs.begin(), fs.end(), [](const Field& a, const Field& b) {
                return a.chan != b.chan ? a.chan < b.chan : a.shift < b.shift;
            });
            uint32_t* dst = which ? D.cpieceV : D.cpieceK;
            int16_t* first = which ? D.cfirstV : D.cfirstK;
            for (size_t i = 0; i < fs.size(); ++i)
                dst[i] = (uint32_t)(fs[i].byte | (fs[i].pos << 8) | (fs[i].width << 12) | (fs[i].shift << 16));
            size_t f = 0;
            for (int j = 0; j <= d; ++j) {
                while (f < fs.size() && fs[f].chan < j) ++f;
                first[j] = (int16_t)f;
            }
            build_encoder_order(fs, d, which ? D.encpermV : D.encpermK);
        }
        int rc = build_decode_schedule(H, D);
        if (rc != AATC_OK) return set_error(rc, "head %zu: %s", h, "decode schedule exceeds kernel limits");
        D.vq_groups = H.vq_groups;
        for (int g = 0; g < H.vq_groups; ++g)
            for (int k = 0; k < kVqDim; ++k) {
                const int j = H.vq_chan[g * kVqDim + k];
                D.vq_chan[g][k] = (uint8_t)j;
                D.vq_scale[j] = H.vq_scale[j];
                D.vq_rscale[j] = (float)(1.0 / (double)H.vq_scale[j]);
                for (int i = 0; i < kVqSize; ++i)
                    D.vq_cent[g][i][k] = H.vq_cent[((size_t)g * kVqSize + i) * kVqDim + k];
            }
    }
    return AATC_OK;
}

static bool finite_all(const double* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!std::isfinite(p[i])) return false;
    return true;
}

}  // namespace aatc

using namespace aatc;

// ======================================================================================
// C ABI: version / errors
// ======================================================================================
// Attention-optimal key transform ("Spend Bits Where Queries Look", abstract: a
// non-orthogonal transform under which the attention-aware key distortion is the MSE of
// the coefficients).  A key error e costs e^T M_Q e; with c = (k - mu) T an error eps in c
// is e = eps T^{-1}, so T = M_Q^{1/2} R makes the cost |eps|^2 for any orthogonal R, and
// R = the eigenvectors of M_Q^{1/2} Sigma_K M_Q^{1/2} decorrelates the coefficients
// (variances lam = its eigenvalues).  M_Q gets a ridge of 1e-6 of its mean eigenvalue so
// that it is invertible.  Outputs T (row-major, [i][j] = T_ij) and T^{-1}.
static int nova_key_transform(int d, const double* sigma_k, const double* m_q, int sweeps, std::vector<double>& lam,
                              std::vector<double>& T, std::vector<double>& Tinv) {
    const size_t dd = (size_t)d * d;
    std::vector<double> M(dd);
    double tr = 0.0;
    for (int i = 0; i < d; ++i) tr += m_q[(size_t)i * d + i];
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) M[(size_t)i * d + j] = 0.5 * (m_q[(size_t)i * d + j] + m_q[(size_t)j * d + i]);
    for (int i = 0; i < d; ++i) M[(size_t)i * d + i] += 1e-6 * tr / d;
    std::vector<double> w, V;
    int rc = jacobi_eigen(d, M.data(), sweeps, w, V);
    if (rc != AATC_OK) return rc;
    for (int k = 0; k < d; ++k)
        if (!(w[k] > 0.0)) return set_error(AATC_ERR_STATS, "M_Q is not positive definite");
    std::vector<double> Mh(dd, 0.0), Mih(dd, 0.0);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double a = 0.0, b = 0.0;
            for (int k = 0; k < d; ++k) {
                const double vv = V[(size_t)i * d + k] * V[(size_t)j * d + k];
                a += vv * std::sqrt(w[k]);
                b += vv / std::sqrt(w[k]);
            }
            Mh[(size_t)i * d + j] = a;
            Mih[(size_t)i * d + j] = b;
        }
    std::vector<double> A(dd, 0.0), tmp(dd, 0.0);  // A = Mh Sigma_K Mh
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double a = 0.0;
            for (int k = 0; k < d; ++k) a += Mh[(size_t)i * d + k] * sigma_k[(size_t)k * d + j];
            tmp[(size_t)i * d + j] = a;
        }
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double a = 0.0;
            for (int k = 0; k < d; ++k) a += tmp[(size_t)i * d + k] * Mh[(size_t)k * d + j];
            A[(size_t)i * d + j] = a;
        }
    for (int i = 0; i < d; ++i)  // exact symmetry for the eigensolver
        for (int j = i + 1; j < d; ++j) {
            const double s = 0.5 * (A[(size_t)i * d + j] + A[(size_t)j * d + i]);
            A[(size_t)i * d + j] = A[(size_t)j * d + i] = s;
        }
    std::vector<double> R;
    rc = jacobi_eigen(d, A.data(), sweeps, lam, R);
    if (rc != AATC_OK) return rc;
    T.assign(dd, 0.0);
    Tinv.assign(dd, 0.0);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double a = 0.0, b = 0.0;
            for (int k = 0; k < d; ++k) {
                a += Mh[(size_t)i * d + k] * R[(size_t)k * d + j];   // T = Mh R
                b += R[(size_t)k * d + i] * Mih[(size_t)k * d + j];  // T^{-1} = R^T Mih
            }
            T[(size_t)i * d + j] = a;
            Tinv[(size_t)i * d + j] = b;
        }
    return AATC_OK;
}

extern "C" int aatc_version(void) { return AATC_VERSION; }
extern "C" int aatc_layout_version(void) { return AATC_LAYOUT_VERSION; }

extern "C" const char* aatc_status_string(int s) {
    switch (s) {
        case AATC_OK: return "ok";
        case AATC_ERR_INVALID_ARG: return "invalid argument";
        case AATC_ERR_UNSUPPORTED: return "unsupported";
        case AATC_ERR_BUDGET: return "bit budget";
        case AATC_ERR_STATS: return "bad statistics";
        case AATC_ERR_NO_CONVERGENCE: return "no convergence";
        case AATC_ERR_CAPACITY: return "capacity";
        case AATC_ERR_WORKSPACE: return "workspace too small";
        case AATC_ERR_HIP: return "HIP error";
        case AATC_ERR_IO: return "I/O error";
        case AATC_ERR_VERSION: return "version mismatch";
        default: return "unknown status";
    }
}

extern "C" const char* aatc_last_error(void) { return g_last_error.c_str(); }

// ======================================================================================
// C ABI: statistics
// ======================================================================================
extern "C" int aatc_stats_from_samples(int32_t d, const float* K, const float* V, int64_t n,
                                       const float* Q, int64_t nq, double* mu_k, double* mu_v,
                                       double* sigma_k, double* sigma_v, double* m_q,
                                       double* gamma_v) {
    if (d != 64 && d != 128) return set_error(AATC_ERR_INVALID_ARG, "d must be 64 or 128 (got %d)", d);
    if (!K || !V || !Q || !mu_k || !mu_v || !sigma_k || !sigma_v || !m_q || !gamma_v)
        return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n < 2 || nq < 1) return set_error(AATC_ERR_INVALID_ARG, "need n >= 2 samples and nq >= 1 queries");
    for (int64_t i = 0; i < n * d; ++i)
        if (!std::isfinite(K[i]) || !std::isfinite(V[i])) return set_error(AATC_ERR_STATS, "non-finite K/V sample");
    for (int64_t i = 0; i < nq * d; ++i)
        if (!std::isfinite(Q[i])) return set_error(AATC_ERR_STATS, "non-finite query sample");

    // means and centred covariances (1/n)
    for (int which = 0; which < 2; ++which) {
        const float* X = which ? V : K;
        double* mu = which ? mu_v : mu_k;
        double* S = which ? sigma_v : sigma_k;
        std::vector<double> m(d, 0.0);
        for (int64_t i = 0; i < n; ++i)
            for (int j = 0; j < d; ++j) m[j] += X[i * d + j];
        for (int j = 0; j < d; ++j) m[j] /= (double)n, mu[j] = m[j];
        std::vector<double> XT((size_t)d * n);  // centred, channel-major
        for (int64_t i = 0; i < n; ++i)
            for (int j = 0; j < d; ++j) XT[(size_t)j * n + i] = (double)X[i * d + j] - m[j];
        parallel_for(d, [&](int64_t a, unsigned) {
            const double* xa = &XT[(size_t)a * n];
            for (int b = (int)a; b < d; ++b) {
                const double* xb = &XT[(size_t)b * n];
                double s = 0.0;
                for (int64_t i = 0; i < n; ++i) s += xa[i] * xb[i];
                S[a * d + b] = S[b * d + a] = s / (double)n;
            }
        });
    }

    // attention-weighted query moment and value weight (exact calibration attention)
    unsigned nw = n_workers();
    std::vector<std::vector<double>> MQp(nw, std::vector<double>((size_t)d * d, 0.0));
    std::vector<double> gp(nw, 0.0);
    std::vector<double> Kd((size_t)n * d), Vd((size_t)n * d);
    for (int64_t i = 0; i < n * d; ++i) Kd[i] = K[i], Vd[i] = V[i];
    const double rs = 1.0 / std::sqrt((double)d);
    parallel_for(nq, [&](int64_t qi, unsigned t) {
        std::vector<double> s(n), o(d, 0.0);
        const float* q = Q + qi * d;
        double qd[kMaxD];
        for (int j = 0; j < d; ++j) qd[j] = q[j];
        double mx = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            const double* k = &Kd[(size_t)i * d];
            for (int j = 0; j < d; ++j) acc += qd[j] * k[j];
            s[i] = acc * rs;
            mx = std::max(mx, s[i]);
        }
        double z = 0.0;
        for (int64_t i = 0; i < n; ++i) z += (s[i] = std::exp(s[i] - mx));
        for (int64_t i = 0; i < n; ++i) s[i] /= z;
        for (int64_t i = 0; i < n; ++i) {
            const double* v = &Vd[(size_t)i * d];
            for (int j = 0; j < d; ++j) o[j] += s[i] * v[j];
        }
        double g = 0.0, a2 = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double* v = &Vd[(size_t)i * d];
            double r = 0.0;
            for (int j = 0; j < d; ++j) r += (v[j] - o[j]) * (v[j] - o[j]);
            g += s[i] * s[i] * r;
            a2 += s[i] * s[i];
        }
        std::vector<double>& M = MQp[t];
        for (int a = 0; a < d; ++a)
            for (int b = 0; b < d; ++b) M[(size_t)a * d + b] += g * qd[a] * qd[b];
        gp[t] += a2;
    });
    for (int i = 0; i < d * d; ++i) {
        double s = 0.0;
        for (unsigned t = 0; t < nw; ++t) s += MQp[t][i];
        m_q[i] = s / (double)nq;
    }
    double g = 0.0;
    for (unsigned t = 0; t < nw; ++t) g += gp[t];
    *gamma_v = g / (double)nq;
    return AATC_OK;
}

// ======================================================================================
// C ABI: calibration
// ======================================================================================
extern "C" int aatc_calibrate(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                              const aatc_head_stats* stats, const aatc_calib_params* p,
                              aatc_codebook** out) {
    if (!out || !stats || !p) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    *out = nullptr;
    if (d != 64 && d != 128) return set_error(AATC_ERR_INVALID_ARG, "d must be 64 or 128 (got %d)", d);
    if (n_layers < 1 || n_kv < 1 || group < 1 || group > 16)
        return set_error(AATC_ERR_INVALID_ARG, "need n_layers >= 1, n_kv >= 1, 1 <= group <= 16");
    int max_bits = p->max_bits ? p->max_bits : 8;
    if (max_bits < 1 || max_bits > 8) return set_error(AATC_ERR_INVALID_ARG, "max_bits must be in [1,8]");
    double totf = 2.0 * d * p->avg_bits;
    int total = (int)std::llround(totf);
    if (!(p->avg_bits > 0) || std::fabs(totf - total) > 1e-9 || total % 8 || total > 2 * d * max_bits)
        return set_error(AATC_ERR_BUDGET, "2*d*avg_bits = %g must be a multiple of 8 in (0, %d]", totf, 2 * d * max_bits);
    if (!p->joint && (total / 2) % kKeyAlign)
        return set_error(AATC_ERR_BUDGET, "separate key/value budgets need d*avg_bits (%d) to be a multiple of %d",
                         total / 2, kKeyAlign);
    const int sweeps = p->max_sweeps > 0 ? p->max_sweeps : 60;
    if (p->key_transform != 0 && p->key_transform != 1)
        return set_error(AATC_ERR_INVALID_ARG, "key_transform must be 0 (KLT) or 1 (attention-optimal)");
    if (p->key_quantizer != 0 && p->key_quantizer != 1)
        return set_error(AATC_ERR_INVALID_ARG, "key_quantizer must be 0 (scalar) or 1 (vector)");
    const int vq_n_g = p->key_quantizer ? total / 2 / 8 : 0;
    if (p->key_quantizer) {
        if (p->joint) return set_error(AATC_ERR_BUDGET, "vector-quantized keys take separate budgets (joint = 0)");
        if (kVqDim * vq_n_g > d)
            return set_error(AATC_ERR_BUDGET, "vector-quantized keys code at most 2 bits per element (avg_bits %g)",
                             p->avg_bits);
        if (!p->vq_normals || p->vq_n_train < kVqSize)
            return set_error(AATC_ERR_INVALID_ARG, "vector-quantized keys need at least %d training draws", kVqSize);
        if (!finite_all(p->vq_normals, (size_t)p->vq_n_train * kVqDim))
            return set_error(AATC_ERR_INVALID_ARG, "non-finite training draw");
        if (p->vq_iters < 0) return set_error(AATC_ERR_INVALID_ARG, "vq_iters must be >= 0");
    }
    const int vq_iters = p->vq_iters > 0 ? p->vq_iters : 20;
    const int n_heads = n_layers * n_kv;

    auto* cb = new aatc_codebook();
    cb->d = d;
    cb->n_layers = n_layers;
    cb->n_kv = n_kv;
    cb->group = group;
    cb->avg_bits = p->avg_bits;
    cb->max_bits = max_bits;
    cb->joint = p->joint ? 1 : 0;
    cb->heads.resize(n_heads);
    std::vector<int> status(n_heads, AATC_OK);
    std::vector<std::string> msg(n_heads);
    const double* steps = step_table();

    parallel_for(n_heads, [&](int64_t h, unsigned) {
        const aatc_head_stats& S = stats[h];
        HeadCB& H = cb->heads[h];
        if (!S.mu_k || !S.mu_v || !S.sigma_k || !S.sigma_v || !S.m_q) {
            status[h] = AATC_ERR_INVALID_ARG;
            msg[h] = "null statistics pointer";
            return;
        }
        if (!finite_all(S.mu_k, d) || !finite_all(S.mu_v, d) || !finite_all(S.sigma_k, (size_t)d * d) ||
            !finite_all(S.sigma_v, (size_t)d * d) || !finite_all(S.m_q, (size_t)d * d) ||
            !std::isfinite(S.gamma_v) || S.gamma_v < 0) {
            status[h] = AATC_ERR_STATS;
            msg[h] = "non-finite statistics";
            return;
        }
        int rc = AATC_OK;
        std::vector<double> Tinv;  // attention-optimal transform only: T^{-1}
        if (p->key_transform == 1) {
            rc = nova_key_transform(d, S.sigma_k, S.m_q, sweeps, H.lamK, H.UK, Tinv);
        } else {
            rc = jacobi_eigen(d, S.sigma_k, sweeps, H.lamK, H.UK);
        }
        if (rc == AATC_OK) rc = jacobi_eigen(d, S.sigma_v, sweeps, H.lamV, H.UV);
        if (rc != AATC_OK) {
            status[h] = rc;
            msg[h] = aatc_last_error();
            return;
        }
        // a PSD covariance has no significantly negative eigenvalue (clamped to 0 above)
        H.muK.assign(S.mu_k, S.mu_k + d);
        H.muV.assign(S.mu_v, S.mu_v + d);
        H.xK.assign(d, 0.0);
        H.xV.assign(d, 0.0);
        for (int j = 0; j < d; ++j) {
            // key weight: coefficient variance x (T^{-1} M_Q T^{-T})_jj / d, with T^{-1} = U_K^T
            // for the KLT (row j of T^{-1} = column j of U_K)
            double w = 0.0;
            for (int a = 0; a < d; ++a) {
                double ua = Tinv.empty() ? H.UK[(size_t)a * d + j] : Tinv[(size_t)j * d + a];
                if (ua == 0.0) continue;
                double r = 0.0;
                for (int b = 0; b < d; ++b)
                    r += S.m_q[(size_t)a * d + b] * (Tinv.empty() ? H.UK[(size_t)b * d + j] : Tinv[(size_t)j * d + b]);
                w += ua * r;
            }
            H.xK[j] = std::max(0.0, H.lamK[j] * w / d);
            H.xV[j] = std::max(0.0, H.lamV[j] * S.gamma_v);
        }
        std::vector<double> xall(H.xK);
        xall.insert(xall.end(), H.xV.begin(), H.xV.end());
        H.theta = waterfill_theta(xall, total, max_bits);
        if (vq_n_g) {
            H.bK.assign(d, 0);
            H.bV = greedy_bits(H.xV, total / 2, max_bits);
            if (!vq_groups(H.xK, vq_n_g, H.vq_chan)) {
                status[h] = AATC_ERR_STATS;
                msg[h] = "a coded key coefficient has zero weight";
                return;
            }
            H.vq_groups = vq_n_g;
            H.vq_scale.assign(d, 0.0f);
            for (int j = 0; j < d; ++j)
                if (H.lamK[j] > 0) H.vq_scale[j] = (float)std::sqrt(std::max(0.0, H.xK[j] / H.lamK[j]));
            H.vq_cent.assign((size_t)vq_n_g * kVqSize * kVqDim, 0.0f);
            const int64_t n = p->vq_n_train;
            std::vector<double> y((size_t)n * kVqDim), code;
            for (int g = 0; g < vq_n_g; ++g) {
                for (int64_t i = 0; i < n; ++i)
                    for (int k = 0; k < kVqDim; ++k)
                        y[(size_t)i * kVqDim + k] =
                            p->vq_normals[(size_t)i * kVqDim + k] * std::sqrt(H.xK[H.vq_chan[g * kVqDim + k]]);
                lloyd(y, n, vq_iters, code);
                for (size_t i = 0; i < code.size(); ++i) H.vq_cent[(size_t)g * kVqSize * kVqDim + i] = (float)code[i];
            }
        } else if (cb->joint) {
            allocate_joint(H.xK, H.xV, total, max_bits, kKeyAlign, H.bK, H.bV);
        } else {
            H.bK = greedy_bits(H.xK, total / 2, max_bits);
            H.bV = greedy_bits(H.xV, total / 2, max_bits);
        }
        H.stepK.assign(d, 0.0f);
        H.stepV.assign(d, 0.0f);
        for (int j = 0; j < d; ++j) {
            if (H.bK[j]) H.stepK[j] = (float)(steps[H.bK[j]] * std::sqrt(H.lamK[j]));
            if (H.bV[j]) H.stepV[j] = (float)(steps[H.bV[j]] * std::sqrt(H.lamV[j]));
        }
    });
    for (int h = 0; h < n_heads; ++h)
        if (status[h] != AATC_OK) {
            delete cb;
            return set_error(status[h], "head %d: %s", h, msg[h].c_str());
        }
    int rc = finalize(cb);
    if (rc != AATC_OK) {
        delete cb;
        return rc;
    }
    *out = cb;
    return AATC_OK;
}

extern "C" int aatc_codebook_create(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                                    const double* U_k, const double* U_v, const double* mu_k,
                                    const double* mu_v, const int32_t* bits_k, const int32_t* bits_v,
                                    const float* step_k, const float* step_v, aatc_codebook** out) {
    if (!out) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    *out = nullptr;
    if (d != 64 && d != 128) return set_error(AATC_ERR_INVALID_ARG, "d must be 64 or 128 (got %d)", d);
    if (n_layers < 1 || n_kv < 1 || group < 1 || group > 16)
        return set_error(AATC_ERR_INVALID_ARG, "need n_layers >= 1, n_kv >= 1, 1 <= group <= 16");
    if (!U_k || !U_v || !mu_k || !mu_v || !bits_k || !bits_v || !step_k || !step_v)
        return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    const int n_heads = n_layers * n_kv;
    auto* cb = new aatc_codebook();
    cb->d = d;
    cb->n_layers = n_layers;
    cb->n_kv = n_kv;
    cb->group = group;
    cb->heads.resize(n_heads);
    const size_t dd = (size_t)d * d;
    for (int h = 0; h < n_heads; ++h) {
        HeadCB& H = cb->heads[h];
        H.UK.assign(U_k + h * dd, U_k + (h + 1) * dd);
        H.UV.assign(U_v + h * dd, U_v + (h + 1) * dd);
        H.muK.assign(mu_k + (size_t)h * d, mu_k + (size_t)(h + 1) * d);
        H.muV.assign(mu_v + (size_t)h * d, mu_v + (size_t)(h + 1) * d);
        H.bK.assign(bits_k + (size_t)h * d, bits_k + (size_t)(h + 1) * d);
        H.bV.assign(bits_v + (size_t)h * d, bits_v + (size_t)(h + 1) * d);
        H.stepK.assign(step_k + (size_t)h * d, step_k + (size_t)(h + 1) * d);
        H.stepV.assign(step_v + (size_t)h * d, step_v + (size_t)(h + 1) * d);
        if (!finite_all(H.UK.data(), dd) || !finite_all(H.UV.data(), dd) || !finite_all(H.muK.data(), d) ||
            !finite_all(H.muV.data(), d)) {
            delete cb;
            return set_error(AATC_ERR_INVALID_ARG, "head %d: non-finite basis or mean", h);
        }
    }
    int rc = finalize(cb);
    if (rc != AATC_OK) {
        delete cb;
        return rc;
    }
    cb->avg_bits = cb->total_bits / (2.0 * d);
    *out = cb;
    return AATC_OK;
}

template <class T, class S>
static void copy_out(T* dst, const std::vector<S>& src) {
    if (dst)
        for (size_t i = 0; i < src.size(); ++i) dst[i] = (T)src[i];
}

extern "C" int aatc_codebook_create_vq(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                                       const double* U_k, const double* U_v, const double* mu_k,
                                       const double* mu_v, int32_t n_groups, const int32_t* vq_chan,
                                       const float* vq_scale, const float* vq_cent, const int32_t* bits_v,
                                       const float* step_v, aatc_codebook** out) {
    if (!out) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    *out = nullptr;
    if (d != 64 && d != 128) return set_error(AATC_ERR_INVALID_ARG, "d must be 64 or 128 (got %d)", d);
    if (n_layers < 1 || n_kv < 1 || group < 1 || group > 16)
        return set_error(AATC_ERR_INVALID_ARG, "need n_layers >= 1, n_kv >= 1, 1 <= group <= 16");
    if (!U_k || !U_v || !mu_k || !mu_v || !vq_chan || !vq_scale || !vq_cent || !bits_v || !step_v)
        return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_groups < 4 || n_groups % 4 || kVqDim * n_groups > d)
        return set_error(AATC_ERR_BUDGET, "n_groups must be a positive multiple of 4 with 4*n_groups <= d");
    const int n_heads = n_layers * n_kv;
    auto* cb = new aatc_codebook();
    cb->d = d;
    cb->n_layers = n_layers;
    cb->n_kv = n_kv;
    cb->group = group;
    cb->joint = 0;
    cb->heads.resize(n_heads);
    const size_t dd = (size_t)d * d, nc = (size_t)n_groups * kVqSize * kVqDim;
    for (int h = 0; h < n_heads; ++h) {
        HeadCB& H = cb->heads[h];
        H.UK.assign(U_k + h * dd, U_k + (h + 1) * dd);
        H.UV.assign(U_v + h * dd, U_v + (h + 1) * dd);
        H.muK.assign(mu_k + (size_t)h * d, mu_k + (size_t)(h + 1) * d);
        H.muV.assign(mu_v + (size_t)h * d, mu_v + (size_t)(h + 1) * d);
        H.bK.assign(d, 0);
        H.stepK.assign(d, 0.0f);
        H.bV.assign(bits_v + (size_t)h * d, bits_v + (size_t)(h + 1) * d);
        H.stepV.assign(step_v + (size_t)h * d, step_v + (size_t)(h + 1) * d);
        H.vq_groups = n_groups;
        H.vq_chan.assign(vq_chan + (size_t)h * kVqDim * n_groups, vq_chan + (size_t)(h + 1) * kVqDim * n_groups);
        H.vq_scale.assign(d, 0.0f);
        for (int32_t j : H.vq_chan)
            if (j >= 0 && j < d) H.vq_scale[j] = vq_scale[(size_t)h * d + j];
        H.vq_cent.assign(vq_cent + h * nc, vq_cent + (h + 1) * nc);
        if (!finite_all(H.UK.data(), dd) || !finite_all(H.UV.data(), dd) || !finite_all(H.muK.data(), d) ||
            !finite_all(H.muV.data(), d)) {
            delete cb;
            return set_error(AATC_ERR_INVALID_ARG, "head %d: non-finite basis or mean", h);
        }
    }
    int rc = finalize(cb);
    if (rc != AATC_OK) {
        delete cb;
        return rc;
    }
    cb->avg_bits = cb->total_bits / (2.0 * d);
    *out = cb;
    return AATC_OK;
}

extern "C" int aatc_codebook_vq(const aatc_codebook* cb, int32_t head, int32_t* n_groups, int32_t* vq_chan,
                                float* vq_scale, float* vq_cent) {
    if (!cb || !n_groups) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (head < 0 || head >= (int)cb->heads.size()) return set_error(AATC_ERR_INVALID_ARG, "head %d out of range", head);
    const HeadCB& H = cb->heads[head];
    *n_groups = H.vq_groups;
    if (H.vq_groups) {
        copy_out(vq_chan, H.vq_chan);
        copy_out(vq_scale, H.vq_scale);
        copy_out(vq_cent, H.vq_cent);
    }
    return AATC_OK;
}

extern "C" int aatc_codebook_info(const aatc_codebook* cb, int32_t* d, int32_t* n_layers, int32_t* n_kv,
                                  int32_t* group, int32_t* total_bits, int32_t* tile_bytes) {
    if (!cb) return set_error(AATC_ERR_INVALID_ARG, "null codebook");
    if (d) *d = cb->d;
    if (n_layers) *n_layers = cb->n_layers;
    if (n_kv) *n_kv = cb->n_kv;
    if (group) *group = cb->group;
    if (total_bits) *total_bits = cb->total_bits;
    if (tile_bytes) *tile_bytes = 8 * cb->total_bits;
    return AATC_OK;
}

extern "C" int aatc_codebook_head(const aatc_codebook* cb, int32_t head, double* U_k, double* U_v,
                                  double* lam_k, double* lam_v, double* mu_k, double* mu_v, double* x_k,
                                  double* x_v, int32_t* bits_k, int32_t* bits_v, float* step_k,
                                  float* step_v, double* theta) {
    if (!cb) return set_error(AATC_ERR_INVALID_ARG, "null codebook");
    if (head < 0 || head >= (int)cb->heads.size()) return set_error(AATC_ERR_INVALID_ARG, "head %d out of range", head);
    const HeadCB& H = cb->heads[head];
    const int d = cb->d;
    copy_out(U_k, H.UK);
    copy_out(U_v, H.UV);
    if (lam_k) std::fill(lam_k, lam_k + d, 0.0), copy_out(lam_k, H.lamK);
    if (lam_v) std::fill(lam_v, lam_v + d, 0.0), copy_out(lam_v, H.lamV);
    copy_out(mu_k, H.muK);
    copy_out(mu_v, H.muV);
    if (x_k) std::fill(x_k, x_k + d, 0.0), copy_out(x_k, H.xK);
    if (x_v) std::fill(x_v, x_v + d, 0.0), copy_out(x_v, H.xV);
    copy_out(bits_k, H.bK);
    copy_out(bits_v, H.bV);
    copy_out(step_k, H.stepK);
    copy_out(step_v, H.stepV);
    if (theta) *theta = H.theta;
    return AATC_OK;
}

extern "C" int aatc_codebook_fields(const aatc_codebook* cb, int32_t head, int32_t which, uint32_t* out,
                                    int32_t* n) {
    if (!cb || !n) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (head < 0 || head >= (int)cb->heads.size()) return set_error(AATC_ERR_INVALID_ARG, "head %d out of range", head);
    if (which != 0 && which != 1) return set_error(AATC_ERR_INVALID_ARG, "which must be 0 (keys) or 1 (values)");
    const std::vector<Field>& fs = which ? cb->heads[head].fV : cb->heads[head].fK;
    *n = (int32_t)fs.size();
    if (out)
        for (size_t i = 0; i < fs.size(); ++i)
            out[i] = (uint32_t)(fs[i].chan | (fs[i].width << 8) | (fs[i].shift << 12) | (fs[i].pos << 16) |
                                (fs[i].byte << 20));
    return AATC_OK;
}

extern "C" void aatc_codebook_free(aatc_codebook* cb) { delete cb; }

// ======================================================================================
// persistence: "AATCCB\0\1" magic, format/layout versions, geometry, per-head arrays,
// FNV-1a 64 checksum of everything before it
// ======================================================================================
namespace {
struct Writer {
    std::vector<uint8_t> buf;
    template <class T>
    void put(const T& v) {
        const uint8_t* p = (const uint8_t*)&v;
        buf.insert(buf.end(), p, p + sizeof(T));
    }
    template <class T>
    void vec(const std::vector<T>& v, size_t n) {
        for (size_t i = 0; i < n; ++i) put<T>(i < v.size() ? v[i] : T(0));
    }
};
struct Reader {
    const uint8_t* p;
    size_t n, at = 0;
    bool ok = true;
    template <class T>
    T get() {
        T v{};
        if (at + sizeof(T) > n) {
            ok = false;
            return v;
        }
        std::memcpy(&v, p + at, sizeof(T));
        at += sizeof(T);
        return v;
    }
    template <class T>
    void vec(std::vector<T>& v, size_t cnt) {
        v.resize(cnt);
        for (size_t i = 0; i < cnt; ++i) v[i] = get<T>();
    }
};
uint64_t fnv1a(const uint8_t* p, size_t n) {
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ p[i]) * 1099511628211ull;
    return h;
}
const char kMagic[8] = {'A', 'A', 'T', 'C', 'C', 'B', 0, 1};
}  // namespace

extern "C" int aatc_codebook_save(const aatc_codebook* cb, const char* path) {
    if (!cb || !path) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    for (const HeadCB& H : cb->heads)
        if (H.vq_groups) return set_error(AATC_ERR_UNSUPPORTED, "codebooks with vector-quantized keys are not persisted");
    Writer w;
    for (char c : kMagic) w.put(c);
    w.put<int32_t>(AATC_VERSION);
    w.put<int32_t>(AATC_LAYOUT_VERSION);
    w.put<int32_t>(cb->d);
    w.put<int32_t>(cb->n_layers);
    w.put<int32_t>(cb->n_kv);
    w.put<int32_t>(cb->group);
    w.put<int32_t>(cb->max_bits);
    w.put<int32_t>(cb->joint);
    w.put<double>(cb->avg_bits);
    const size_t d = cb->d, dd = d * d;
    for (const HeadCB& H : cb->heads) {
        w.vec(H.UK, dd);
        w.vec(H.UV, dd);
        w.vec(H.lamK, d);
        w.vec(H.lamV, d);
        w.vec(H.muK, d);
        w.vec(H.muV, d);
        w.vec(H.xK, d);
        w.vec(H.xV, d);
        w.vec(H.bK, d);
        w.vec(H.bV, d);
        w.vec(H.stepK, d);
        w.vec(H.stepV, d);
        w.put<double>(H.theta);
    }
    w.put<uint64_t>(fnv1a(w.buf.data(), w.buf.size()));
    FILE* f = std::fopen(path, "wb");
    if (!f) return set_error(AATC_ERR_IO, "cannot open %s for writing", path);
    size_t wr = std::fwrite(w.buf.data(), 1, w.buf.size(), f);
    int cl = std::fclose(f);
    if (wr != w.buf.size() || cl != 0) return set_error(AATC_ERR_IO, "short write to %s", path);
    return AATC_OK;
}

extern "C" int aatc_codebook_load(const char* path, aatc_codebook** out) {
    if (!path || !out) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    *out = nullptr;
    FILE* f = std::fopen(path, "rb");
    if (!f) return set_error(AATC_ERR_IO, "cannot open %s", path);
    std::vector<uint8_t> buf;
    uint8_t tmp[65536];
    size_t r;
    while ((r = std::fread(tmp, 1, sizeof tmp, f)) > 0) buf.insert(buf.end(), tmp, tmp + r);
    std::fclose(f);
    if (buf.size() < 8 + 8 * 4 + 8 + 8 || std::memcmp(buf.data(), kMagic, 8) != 0)
        return set_error(AATC_ERR_VERSION, "%s is not a codebook file", path);
    uint64_t stored;
    std::memcpy(&stored, buf.data() + buf.size() - 8, 8);
    if (fnv1a(buf.data(), buf.size() - 8) != stored) return set_error(AATC_ERR_VERSION, "%s: checksum mismatch", path);
    Reader rd{buf.data(), buf.size() - 8};
    rd.at = 8;
    int ver = rd.get<int32_t>(), lay = rd.get<int32_t>();
    if (ver != AATC_VERSION || lay != AATC_LAYOUT_VERSION)
        return set_error(AATC_ERR_VERSION, "%s: format %d/layout %d, library %d/%d", path, ver, lay, AATC_VERSION,
                         AATC_LAYOUT_VERSION);
    auto* cb = new aatc_codebook();
    cb->d = rd.get<int32_t>();
    cb->n_layers = rd.get<int32_t>();
    cb->n_kv = rd.get<int32_t>();
    cb->group = rd.get<int32_t>();
    cb->max_bits = rd.get<int32_t>();
    cb->joint = rd.get<int32_t>();
    cb->avg_bits = rd.get<double>();
    if (!rd.ok || (cb->d != 64 && cb->d != 128) || cb->n_layers < 1 || cb->n_kv < 1 || cb->n_layers * (int64_t)cb->n_kv > (1 << 20)) {
        delete cb;
        return set_error(AATC_ERR_VERSION, "%s: bad header", path);
    }
    const size_t d = cb->d, dd = d * d;
    cb->heads.resize((size_t)cb->n_layers * cb->n_kv);
    for (HeadCB& H : cb->heads) {
        rd.vec(H.UK, dd);
        rd.vec(H.UV, dd);
        rd.vec(H.lamK, d);
        rd.vec(H.lamV, d);
        rd.vec(H.muK, d);
        rd.vec(H.muV, d);
        rd.vec(H.xK, d);
        rd.vec(H.xV, d);
        rd.vec(H.bK, d);
        rd.vec(H.bV, d);
        rd.vec(H.stepK, d);
        rd.vec(H.stepV, d);
        H.theta = rd.get<double>();
    }
    if (!rd.ok || rd.at != rd.n) {
        delete cb;
        return set_error(AATC_ERR_VERSION, "%s: truncated or oversized file", path);
    }
    int rc = finalize(cb);
    if (rc != AATC_OK) {
        delete cb;
        return rc;
    }
    *out = cb;
    return AATC_OK;
}
