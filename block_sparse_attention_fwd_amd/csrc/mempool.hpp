// Recycling memory pools for plans.
//
// A dynamic mask is planned per request, so every request would otherwise pay
// for a fresh pinned host buffer, a fresh device buffer and the page faults of
// first touching them. Plans instead take blocks from these pools and return
// them when destroyed. Blocks are reused best-fit within a 1.5x size window;
// cached bytes are capped and the largest blocks are released first when the
// cap is exceeded.
#pragma once

#include <cstddef>
#include <functional>
#include <map>
#include <mutex>

namespace bsa {

class BlockPool {
  public:
    using AllocFn = std::function<void *(size_t)>;  // nullptr on failure
    using FreeFn = std::function<void(void *)>;

    BlockPool(AllocFn alloc, FreeFn release, size_t cap_bytes)
        : alloc_(std::move(alloc)), free_(std::move(release)), cap_(cap_bytes) {}

    // A block of at least `want` bytes; its usable size goes to *got.
    void *acquire(size_t want, size_t *got)
    {
        want = round(want);
        {
            std::lock_guard<std::mutex> g(mu_);
            auto it = cached_.lower_bound(want);
            if (it != cached_.end() && it->first <= want + want / 2) {
                void *p = it->second;
                *got = it->first;
                cached_bytes_ -= it->first;
                cached_.erase(it);
                return p;
            }
        }
        void *p = alloc_(want);
        if (!p) {
            trim(0);  // give cached memory back and try once more
            p = alloc_(want);
        }
        *got = p ? want : 0;
        return p;
    }

    void release(void *p, size_t size)
    {
        if (!p) return;
        {
            std::lock_guard<std::mutex> g(mu_);
            cached_.emplace(size, p);
            cached_bytes_ += size;
        }
        trim(cap_);
    }

    // Free cached blocks (largest first) until at most `keep` bytes remain.
    void trim(size_t keep)
    {
        for (;;) {
            void *p = nullptr;
            {
                std::lock_guard<std::mutex> g(mu_);
                if (cached_bytes_ <= keep || cached_.empty()) return;
                auto it = std::prev(cached_.end());
                p = it->second;
                cached_bytes_ -= it->first;
                cached_.erase(it);
            }
            free_(p);
        }
    }

  private:
    static size_t round(size_t n)
    {
        const size_t g = 64 * 1024;
        return ((n ? n : 1) + g - 1) / g * g;
    }

    AllocFn alloc_;
    FreeFn free_;
    size_t cap_;
    std::mutex mu_;
    std::multimap<size_t, void *> cached_;
    size_t cached_bytes_ = 0;
};

}  // namespace bsa
