// Host model of one 64-lane wave running walk_pieces_any (wave_walk.h, the
// piece walk of the a2av copy for more than 8 ranks), the very code the GPU
// kernel runs: 64 threads, one per lane, in lockstep at every cross-lane
// operation. The model stops the program (exit code 3 or 4) when a cross-lane
// operation is not reached by every lane, or lanes reach different ones; when
// a value said to be the same in every lane is not (4); and when a load or a
// copy leaves the buffers it may touch (5).
//
// Usage: wave_walk_host CASE_FILE OUT_FILE
// CASE_FILE (little-endian): int64 W, R, piece, waves; int64 in_rows[W],
// cap[W], recv_off[W][W+1], send_off[W][W+1]; then the input bytes of ranks
// 0..W-1 (in_rows[s] * R each).
// OUT_FILE: the output bytes of ranks 0..W-1 (cap[d] * R each, starting as
// 0xA5), then one byte per output byte: how many copies wrote it (saturating
// at 255).
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <unistd.h>
#include <vector>

#include "wave_walk.h"

namespace {

constexpr int kLanes = 64;

[[noreturn]] void die(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vfprintf(stderr, fmt, ap);
    va_end(ap);
    std::fputc('\n', stderr);
    std::fflush(stderr);
    _exit(code);
}

struct Args {
    int W;
    uint64_t R, piece;
    const unsigned char *in[64];
    unsigned char *out[64];
    int64_t in_rows[64], cap[64];
    const int64_t *recv_off, *send_off;
};

struct Range {
    const unsigned char *lo;
    uint64_t bytes;
};

struct Shared {
    std::atomic<int> arrived{0};
    std::atomic<uint64_t> gen{0};
    uint64_t val[kLanes];
    int site[kLanes];
    std::vector<Range> matrices, ins, outs;
    std::vector<unsigned char> *count = nullptr;  // writes per output byte
    const unsigned char *out_base = nullptr;
    uint64_t copies = 0;
};

bool inside(const std::vector<Range> &rs, const void *p, uint64_t n) {
    const unsigned char *c = (const unsigned char *)p;
    for (const Range &r : rs)
        if (c >= r.lo && n <= r.bytes && (uint64_t)(c - r.lo) <= r.bytes - n) return true;
    return false;
}

// A barrier of the 64 lane threads: the last to arrive opens the next
// generation; the others yield until it does, and give up after 20 s (a lane
// that never arrives: the lanes diverged).
void sync(Shared &sh) {
    const uint64_t g = sh.gen.load(std::memory_order_acquire);
    if (sh.arrived.fetch_add(1, std::memory_order_acq_rel) == kLanes - 1) {
        sh.arrived.store(0, std::memory_order_relaxed);
        sh.gen.store(g + 1, std::memory_order_release);
        return;
    }
    const auto t0 = std::chrono::steady_clock::now();
    for (unsigned spin = 0; sh.gen.load(std::memory_order_acquire) == g; spin++) {
        std::this_thread::yield();
        if ((spin & 1023) == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20))
            die(3, "a cross-lane operation was not reached by every lane");
    }
}

class HostWave {
  public:
    HostWave(int lane, Shared &sh) : ln_(lane), sh_(sh) {}
    int lane() const { return ln_; }
    int64_t load(const int64_t *p) {
        if (!inside(sh_.matrices, p, 8)) die(5, "lane %d loads outside the offset matrices", ln_);
        return *p;
    }
    int64_t load_uniform(const int64_t *p) {
        same(100, (uint64_t)(uintptr_t)p, "load_uniform address");
        return load(p);
    }
    void copy(unsigned char *d, const unsigned char *s, uint64_t n) {
        same(101, (uint64_t)(uintptr_t)d, "copy destination");
        same(102, (uint64_t)(uintptr_t)s, "copy source");
        same(103, n, "copy length");
        if (ln_ != 0) return;
        if (!inside(sh_.outs, d, n)) die(5, "a copy of %llu bytes writes outside the outputs",
                                         (unsigned long long)n);
        if (!inside(sh_.ins, s, n)) die(5, "a copy of %llu bytes reads outside the inputs",
                                        (unsigned long long)n);
        std::memcpy(d, s, n);
        for (uint64_t i = 0; i < n; i++) {
            unsigned char &c = (*sh_.count)[(uint64_t)(d - sh_.out_base) + i];
            if (c < 255) c++;
        }
        sh_.copies++;
    }
    uint64_t ballot(int site, bool b) {
        return exchange(site, b ? 1 : 0, [](const uint64_t *v, int) {
            uint64_t m = 0;
            for (int i = 0; i < kLanes; i++) m |= (v[i] & 1) << i;
            return m;
        });
    }
    uint64_t readlane(int site, uint64_t v, int l) {
        same(site + 1000, (uint64_t)l, "readlane index");
        if (l < 0 || l >= kLanes) die(4, "readlane index %d", l);
        return exchange(site, v, [l](const uint64_t *x, int) { return x[l]; });
    }
    int uniform(int site, int x) { return (int)same(site, (uint64_t)(int64_t)x, "uniform value"); }
    uint64_t dest_totals(int site, const Args &a) {
        same(site, 0, "destination totals");
        return ln_ < a.W ? (uint64_t)load(a.recv_off + (uint64_t)ln_ * (a.W + 1) + a.W) : 0;
    }
    void row(int site, const Args &a, int d, uint64_t &ro, uint64_t &n) {
        same(site, (uint64_t)(int64_t)d, "row destination");
        if (d < 0 || d >= a.W) die(4, "row of destination %d", d);
        const int64_t *rrow = a.recv_off + (uint64_t)d * (a.W + 1);
        ro = ln_ < a.W ? (uint64_t)load(rrow + ln_) : 0;
        n = ln_ < a.W ? (uint64_t)load(rrow + ln_ + 1) - ro : 0;
    }
    uint64_t incl_scan(int site, uint64_t v) {
        return exchange(site, v, [](const uint64_t *x, int lane) {
            uint64_t s = 0;
            for (int i = 0; i <= lane; i++) s += x[i];
            return s;
        });
    }

  private:
    template <class F>
    uint64_t exchange(int site, uint64_t v, F f) {
        sh_.val[ln_] = v;
        sh_.site[ln_] = site;
        sync(sh_);
        for (int i = 0; i < kLanes; i++)
            if (sh_.site[i] != site)
                die(4, "lane %d is at cross-lane operation %d while lane %d is at %d", ln_, site, i,
                    sh_.site[i]);
        const uint64_t r = f(sh_.val, ln_);
        sync(sh_);
        return r;
    }
    uint64_t same(int site, uint64_t v, const char *what) {
        return exchange(site, v, [&](const uint64_t *x, int) {
            for (int i = 1; i < kLanes; i++)
                if (x[i] != x[0]) die(4, "%s differs between lanes 0 and %d", what, i);
            return x[0];
        });
    }
    int ln_;
    Shared &sh_;
};

std::vector<int64_t> read_i64(FILE *f, size_t n) {
    std::vector<int64_t> v(n);
    if (n && std::fread(v.data(), 8, n, f) != n) die(2, "short case file");
    return v;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 3) die(2, "usage: wave_walk_host CASE_FILE OUT_FILE");
    FILE *f = std::fopen(argv[1], "rb");
    if (!f) die(2, "cannot open %s", argv[1]);
    const std::vector<int64_t> hdr = read_i64(f, 4);
    const int W = (int)hdr[0];
    if (W < 1 || W > 64) die(2, "W = %d", W);
    Args a{};
    a.W = W;
    a.R = (uint64_t)hdr[1];
    a.piece = (uint64_t)hdr[2];
    const uint64_t waves = (uint64_t)hdr[3];
    const std::vector<int64_t> in_rows = read_i64(f, W), cap = read_i64(f, W);
    const std::vector<int64_t> recv_off = read_i64(f, (size_t)W * (W + 1));
    const std::vector<int64_t> send_off = read_i64(f, (size_t)W * (W + 1));
    Shared sh;
    std::vector<std::vector<unsigned char>> in(W);
    uint64_t out_total = 0;
    for (int r = 0; r < W; r++) out_total += (uint64_t)cap[r] * a.R;
    std::vector<unsigned char> out(out_total, 0xA5), count(out_total, 0);
    uint64_t o = 0;
    for (int r = 0; r < W; r++) {
        in[r].resize((uint64_t)in_rows[r] * a.R);
        if (!in[r].empty() && std::fread(in[r].data(), 1, in[r].size(), f) != in[r].size())
            die(2, "short case file");
        a.in[r] = in[r].data();
        a.out[r] = out.data() + o;
        a.in_rows[r] = in_rows[r];
        a.cap[r] = cap[r];
        sh.ins.push_back({a.in[r], in[r].size()});
        sh.outs.push_back({a.out[r], (uint64_t)cap[r] * a.R});
        o += (uint64_t)cap[r] * a.R;
    }
    std::fclose(f);
    a.recv_off = recv_off.data();
    a.send_off = send_off.data();
    sh.matrices.push_back({(const unsigned char *)recv_off.data(), recv_off.size() * 8});
    sh.matrices.push_back({(const unsigned char *)send_off.data(), send_off.size() * 8});
    sh.count = &count;
    sh.out_base = out.data();

    std::vector<std::thread> lanes;
    for (int l = 0; l < kLanes; l++)
        lanes.emplace_back([&, l] {
            for (uint64_t gw = 0; gw < waves; gw++) {
                HostWave wv(l, sh);
                a2av::walk_pieces_any(wv, a, gw, waves);
                sync(sh);  // every lane leaves the wave together
            }
        });
    for (std::thread &t : lanes) t.join();

    FILE *g = std::fopen(argv[2], "wb");
    if (!g) die(2, "cannot open %s", argv[2]);
    if (out_total && (std::fwrite(out.data(), 1, out_total, g) != out_total ||
                      std::fwrite(count.data(), 1, out_total, g) != out_total))
        die(2, "short write");
    std::fclose(g);
    std::printf("copies %llu\n", (unsigned long long)sh.copies);
    return 0;
}
